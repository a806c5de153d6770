"""Parity at the benchmark's full sizes, through the same call the benchmark
times.  For the paper workload (the benchmark's) and the linear workload the
oracle computes every row of g_hat (token by token, in parallel over tokens)
and G_W is compared whole with the fp64 product of the oracle's g_hat and X.
For K = 1024 and 16384 the oracle computes a fixed sample of 128 rows (seed 1)
plus the sequence boundaries, and G_W is checked on sampled rows against the
fp64 outer product of the returned g_hat (the identity G_W = sum_t g_t x_t^T
holds at any size).  Every comparison is made on the whole array, row by row
and element by element (see util)."""
import numpy as np
import pytest

import oracle
from activation_perturbation_estimator_amd import synth
from util import (G_HAT_TERM_TOL, G_W_RSS_TOL, assert_elementwise, assert_gw, assert_parity,
                  assert_rows, gw_rss_scale, need_gpu)

pytestmark = pytest.mark.gpu

SAMPLE_TOKENS = 128


def _sample_tokens(T, L, n, seed=1):
    rng = np.random.default_rng(seed)
    tok = set(rng.choice(T, size=n, replace=False).tolist())
    tok |= {0, L - 1, L, T - 1}
    return np.array(sorted(tok), dtype=np.int64)


def _check_gw_rows(g, X64, G, nrows=48):
    """Rows of G_W against the fp64 outer product of the returned g_hat."""
    rng = np.random.default_rng(2)
    rows = rng.choice(g.shape[1], size=min(nrows, g.shape[1]), replace=False)
    gs = g[:, rows].astype(np.float64)
    ref = gs.T @ X64
    assert_parity(G[rows], ref, "G_W rows")
    assert_elementwise(G[rows], ref, gw_rss_scale(gs, X64), "G_W row elements", G_W_RSS_TOL,
                       atol=1e-6 * float(np.abs(ref).max()))


def _check_g(g, ref, scale, what):
    assert_parity(g, ref, what)
    assert_rows(g, ref, what + " rows")
    assert_elementwise(g, ref, scale, what + " elements", G_HAT_TERM_TOL)


def test_head_paper_every_row():
    dust = need_gpu()
    import torch
    w = synth.WORKLOADS["paper"]
    z, y, X = synth.workload_inputs(w)
    print(f"[fullsize] paper, every row: T={w.T} V={w.V} d={w.d} K={w.K}", flush=True)
    g, G = dust.head_estimate(z.cuda(), y.cuda(), X.cuda(), sigma=w.sigma, K=w.K,
                              gamma=w.gamma, seed=w.philox_seed, seq_len=w.seq_len)
    torch.cuda.synchronize()
    g = g.cpu().numpy()
    G = G.cpu().numpy()
    ref, scale = oracle.head_rows(synth.to_f64(z), y.numpy(), w.seq_len, w.sigma, w.K, w.gamma,
                                  w.philox_seed, np.arange(w.T), with_scale=True)
    _check_g(g, ref, scale, "g_hat, every row")
    del scale
    assert_gw(G, ref, synth.to_f64(X))


@pytest.mark.parametrize("name", ["k1024", "k16384"])
def test_head_full_size(name):
    dust = need_gpu()
    import torch
    w = synth.WORKLOADS[name]
    z, y, X = synth.workload_inputs(w)
    tok = _sample_tokens(w.T, w.seq_len, SAMPLE_TOKENS)
    print(f"[fullsize] {name}: T={w.T} V={w.V} d={w.d} K={w.K}, {len(tok)} sampled rows",
          flush=True)
    g, G = dust.head_estimate(z.cuda(), y.cuda(), X.cuda(), sigma=w.sigma, K=w.K,
                              gamma=w.gamma, seed=w.philox_seed, seq_len=w.seq_len)
    torch.cuda.synchronize()
    g = g.cpu().numpy()
    G = G.cpu().numpy()
    assert np.isfinite(g).all() and np.isfinite(G).all()
    zs = synth.to_f64(z[tok])
    # gamma = 0: a token's row depends only on its own logits and index; the
    # oracle is given the sampled rows placed at their true token indices.
    zfull = np.zeros((w.T, w.V))
    zfull[tok] = zs
    rows, scale = oracle.head_rows(zfull, y.numpy(), w.seq_len, w.sigma, w.K, w.gamma,
                                   w.philox_seed, tok, with_scale=True)
    _check_g(g[tok], rows, scale, "g_hat sampled rows")
    _check_gw_rows(g, synth.to_f64(X), G)


def test_linear_full_size():
    dust = need_gpu()
    import torch
    w = synth.WORKLOADS["linear"]
    X, c = synth.workload_inputs(w)
    print(f"[fullsize] linear: T={w.T} N={w.V} d={w.d} K={w.K} gamma={w.gamma}", flush=True)
    g, G = dust.linear_estimate(X.cuda(), c.cuda(), N=w.V, sigma=w.sigma, gamma=w.gamma,
                                seed=w.philox_seed, seq_len=w.seq_len)
    torch.cuda.synchronize()
    g = g.cpu().numpy()
    G = G.cpu().numpy()
    ref, scale = oracle.linear_rows(c.double().numpy(), w.seq_len, w.V, w.sigma, w.gamma,
                                    w.philox_seed, np.arange(w.T), with_scale=True)
    _check_g(g, ref, scale, "g_hat, every row")
    del scale
    assert_gw(G, ref, synth.to_f64(X))
