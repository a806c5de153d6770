"""Parity at the benchmark's full sizes, through the same call the benchmark
times.  The oracle computes sampled rows of g_hat token by token (plus the
sequence boundaries); G_W is checked on sampled rows against the fp64 outer
product of the returned g_hat (the identity G_W = sum_t g_t x_t^T holds at any
size), and its norm against the sampled-row relation."""
import numpy as np
import pytest

import oracle
from activation_perturbation_estimator_amd import synth
from util import assert_parity, need_gpu

pytestmark = pytest.mark.gpu


def _sample_tokens(T, L, n, seed=1):
    rng = np.random.default_rng(seed)
    tok = set(rng.choice(T, size=n, replace=False).tolist())
    tok |= {0, L - 1, L, T - 1}
    return np.array(sorted(tok), dtype=np.int64)


def _check_gw(g, X64, G, nrows=48):
    rng = np.random.default_rng(2)
    rows = rng.choice(g.shape[1], size=min(nrows, g.shape[1]), replace=False)
    ref = g[:, rows].astype(np.float64).T @ X64
    assert_parity(G[rows], ref, "G_W rows")


@pytest.mark.parametrize("name,ntok", [("paper", 24), ("k1024", 6), ("k16384", 2)])
def test_head_full_size(name, ntok):
    dust = need_gpu()
    import torch
    w = synth.WORKLOADS[name]
    z, y, X = synth.workload_inputs(w)
    print(f"[fullsize] {name}: T={w.T} V={w.V} d={w.d} K={w.K}", flush=True)
    g, G = dust.head_estimate(z.cuda(), y.cuda(), X.cuda(), sigma=w.sigma, K=w.K,
                              gamma=w.gamma, seed=w.philox_seed, seq_len=w.seq_len)
    torch.cuda.synchronize()
    g = g.cpu().numpy()
    G = G.cpu().numpy()
    assert np.isfinite(g).all() and np.isfinite(G).all()
    tok = _sample_tokens(w.T, w.seq_len, ntok)
    zs = synth.to_f64(z[tok])
    # gamma = 0: a token's row depends only on its own logits and index; the
    # oracle is given the sampled rows placed at their true token indices.
    zfull = np.zeros((w.T, w.V))
    zfull[tok] = zs
    rows = oracle.head_rows(zfull, y.numpy(), w.seq_len, w.sigma, w.K, w.gamma, w.philox_seed,
                            tok)
    assert_parity(g[tok], rows, "g_hat sampled rows")
    _check_gw(g, synth.to_f64(X), G)


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
    tok = _sample_tokens(w.T, w.seq_len, 24)
    rows = oracle.linear_rows(c.double().numpy(), w.seq_len, w.V, w.sigma, w.gamma,
                              w.philox_seed, tok)
    assert_parity(g[tok], rows, "g_hat sampled rows")
    _check_gw(g, synth.to_f64(X), G)
