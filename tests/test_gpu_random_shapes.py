"""Seeded random shapes against the oracle, one generator per case (seeded by
the case number):
  - the LM-head and hidden-layer estimates (paper digest, section 2.2): sequence
    length, token count, width, vocabulary, population, discount, sigma, dtypes,
    seed and stream drawn at random; whole arrays and every row of g_hat within
    relative L2 1e-3 and cosine 0.99999, every element of g_hat within 1e-4 of
    its error scale, and G_W against the fp64 product;
  - the outer product over token rows spanning many binades (some left to the
    exact fp32 pass);
  - the reward scan, element by element against the size of what it sums;
  - the embedding estimate, row by row against the size of what it sums;
  - the perturbed forward, element by element against the product's size."""
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


@pytest.mark.parametrize("case", range(12))
def test_outer_sum_random_shape(case):
    """dust_outer_sum on random shapes whose token rows span many binades (the
    per-token power-of-two scaling of the fp16 pass), with some tokens whose
    range no scale fits (left to the exact fp32 pass)."""
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(3000 + case)
    T, N, d = int(rng.integers(1, 6000)), int(rng.integers(1, 1500)), int(rng.integers(1, 700))
    bf16 = bool(rng.integers(0, 2))
    print(f"[random outer sum] case {case}: T={T} N={N} d={d} bf16={bf16}", flush=True)
    g = rng.standard_normal((T, N)) * np.exp2(rng.uniform(-30, 30, (T, 1)))
    g[rng.random(T) < 0.02] *= 2.0**-60  # products below what fp16 holds after scaling
    g = g.astype(np.float32)
    Xf = (rng.standard_normal((T, d)) * np.exp2(rng.uniform(-10, 10, (T, 1)))).astype(np.float32)
    X = torch.from_numpy(Xf).to(torch.bfloat16) if bf16 else torch.from_numpy(Xf)
    G = dust.outer_sum(torch.from_numpy(g).cuda(), X.cuda())
    torch.cuda.synchronize()
    assert_gw(G.cpu().numpy(), g.astype(np.float64), synth.to_f64(X))


@pytest.mark.parametrize("case", range(12))
def test_reward_scan_random_shape(case):
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(4000 + case)
    L = int(rng.choice([1, 2, 5, 63, 64, 255, 256, 1000, 2048, 4097, 9000]))
    T = L * int(rng.integers(1, 4))
    K = int(rng.integers(1, 9))
    gamma = float(rng.choice([0.0, 0.3, 0.9, 1.0]))
    print(f"[random scan] case {case}: K={K} T={T} L={L} gamma={gamma}", flush=True)
    c = rng.standard_normal((K, T)).astype(np.float32)
    r = dust.reward_scan(torch.from_numpy(c).cuda(), seq_len=L, gamma=gamma)
    torch.cuda.synchronize()
    got = r.cpu().numpy()
    if gamma == 0.0:
        assert np.array_equal(got, c)
    else:
        ref = oracle.reward_scan(c.astype(np.float64), L, gamma)
        # per sequence: the recurrence's fp32 rounding against the size of what it sums
        scale = oracle.reward_scan(np.abs(c).astype(np.float64), L, gamma)
        assert (np.abs(got - ref) <= 1e-5 * scale + 1e-30).all()


@pytest.mark.parametrize("case", range(8))
def test_embedding_random_shape(case):
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(5000 + case)
    T, N, vocab = int(rng.integers(1, 40000)), 4 * int(rng.integers(1, 130)), int(rng.integers(1, 9000))
    print(f"[random embedding] case {case}: T={T} N={N} vocab={vocab}", flush=True)
    ids = synth.zipf_targets(rng, T, vocab) if rng.integers(0, 2) else \
        rng.integers(-2, vocab + 2, T).astype(np.int32)
    g = rng.standard_normal((T, N)).astype(np.float32)
    G = dust.embedding_grad(torch.from_numpy(ids).cuda(), torch.from_numpy(g).cuda(), vocab)
    torch.cuda.synchronize()
    G = G.cpu().numpy()
    ref = oracle.embedding_grad(ids, g.astype(np.float64), vocab)
    # each row sums its tokens' rows in fp32: within 1e-5 of the sum of magnitudes
    absref = oracle.embedding_grad(ids, np.abs(g).astype(np.float64), vocab)
    assert (np.abs(G - ref) <= 1e-5 * absref).all()
    assert (G[absref == 0] == 0).all()


@pytest.mark.parametrize("case", range(8))
def test_forward_random_shape(case):
    """The perturbed forward Y[k] = X W^T + sigma a^(draw0+k) on random shapes,
    draw offsets, streams and seeds, element by element: within 1e-4 of the
    product's magnitude sum_j |x_j w_j| plus 1e-5 of sigma (the noise in fp32)."""
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(6000 + case)
    # the call takes d % 8 == 0 and N % 4 == 0
    T, d, N = int(rng.integers(1, 700)), 8 * int(rng.integers(1, 40)), 4 * int(rng.integers(1, 300))
    ndraw, draw0 = int(rng.integers(1, 5)), int(rng.integers(0, 2**31))
    stream, seed = int(rng.integers(0, 2**32)), int(rng.integers(0, 2**63))
    bf16 = bool(rng.integers(0, 2))
    sigma = float(rng.choice([0.01, 0.1, 1.0]))
    print(f"[random forward] case {case}: T={T} d={d} N={N} ndraw={ndraw} bf16={bf16}", flush=True)
    dt = torch.bfloat16 if bf16 else torch.float32
    X = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32) / np.sqrt(d)).to(dt)
    W = torch.from_numpy(rng.standard_normal((N, d)).astype(np.float32) / np.sqrt(d)).to(dt)
    Y = dust.perturbed_linear(X.cuda(), W.cuda(), sigma=sigma, seed=seed, stream=stream,
                              draw0=draw0, ndraw=ndraw)
    torch.cuda.synchronize()
    Xd, Wd = synth.to_f64(X), synth.to_f64(W)
    ref = oracle.perturbed_linear(Xd, Wd, sigma, seed, stream, draw0, ndraw)
    mag = np.abs(Xd) @ np.abs(Wd).T
    assert (np.abs(Y.cpu().numpy() - ref) <= 1e-4 * mag[None] + 1e-5 * sigma).all()
