"""Each GPU stage of the estimator against the oracle (paper digest, section 2.2;
laoyaoba analysis, mechanism section), at sizes that span several tiles and
leave ragged tails.

Tolerances: per-draw losses |error| <= 2e-4 nats (fp32 logsumexp of ~6-nat
losses over up to 16k terms); centring and the scan within fp32 rounding
(relative L2 <= 1e-5; gamma = 0 is bit-exact); error estimate and outer product
relative L2 <= 1e-3 and cosine >= 0.99999."""
import numpy as np
import pytest

import oracle
from activation_perturbation_estimator_amd import synth
from util import assert_parity, need_gpu, rel_l2

pytestmark = pytest.mark.gpu


def _cuda(t):
    return t.contiguous().cuda()


@pytest.mark.parametrize("T,V,K,bf16", [(256, 512, 16, False), (70, 1000, 9, True),
                                         (33, 4096, 65, True), (5, 12, 3, False),
                                         (4, 20000, 3, True), (3, 40000, 2, False)])
def test_head_losses(T, V, K, bf16):
    dust = need_gpu()
    import torch
    z, y, _ = synth.head_inputs(T, V, 4, seed=T + V, bf16=bf16)
    sigma, seed, stream = 0.07, 5, 2
    got = dust.head_losses(_cuda(z), _cuda(y), sigma=sigma, K=K, seed=seed, stream=stream)
    torch.cuda.synchronize()
    _, _, diag = oracle.head_estimate(synth.to_f64(z), y.numpy(), np.zeros((T, 1)), T, sigma, K,
                                      0.0, seed, stream, diagnostics=True)
    err = np.abs(got.cpu().numpy() - diag["ell"])
    assert err.max() <= 2e-4, err.max()


@pytest.mark.parametrize("K,T", [(16, 256), (1, 7), (1000, 33), (3, 5000)])
def test_centre(K, T):
    dust = need_gpu()
    import torch
    x = torch.from_numpy(np.random.default_rng(K).standard_normal((K, T)).astype(np.float32) + 6)
    c = dust.centre(_cuda(x))
    torch.cuda.synchronize()
    xd = x.double().numpy()
    ref = xd.mean(0, keepdims=True) - xd
    assert np.abs(c.cpu().numpy() - ref).max() <= 1e-6
    # in place
    xg = _cuda(x)
    dust.centre(xg, out=xg)
    torch.cuda.synchronize()
    assert np.abs(xg.cpu().numpy() - ref).max() <= 1e-6


@pytest.mark.parametrize("K,T,L", [(3, 60, 1), (2, 70, 7), (2, 1024, 512), (2, 1026, 513),
                                   (3, 4096, 2048), (1, 6000, 3000), (5, 600, 600),
                                   (2, 8200, 4100), (2, 2046, 1023)])
@pytest.mark.parametrize("gamma", [0.0, 0.5, 0.9, 1.0])
def test_reward_scan(K, T, L, gamma):
    dust = need_gpu()
    import torch
    c = np.random.default_rng(T + L).standard_normal((K, T)).astype(np.float32)
    r = dust.reward_scan(_cuda(torch.from_numpy(c)), seq_len=L, gamma=gamma)
    torch.cuda.synchronize()
    got = r.cpu().numpy()
    ref = oracle.reward_scan(c.astype(np.float64), L, gamma)
    if gamma == 0.0:
        assert np.array_equal(got, c)
    else:
        assert rel_l2(got, ref) <= 1e-5, rel_l2(got, ref)


def test_reward_scan_in_place_and_isolation():
    dust = need_gpu()
    import torch
    c = np.random.default_rng(1).standard_normal((2, 3000)).astype(np.float32)
    g = _cuda(torch.from_numpy(c))
    dust.reward_scan(g, seq_len=1000, gamma=0.95, out=g)
    c2 = c.copy()
    c2[1, 1500] += 3.0
    g2 = dust.reward_scan(_cuda(torch.from_numpy(c2)), seq_len=1000, gamma=0.95)
    torch.cuda.synchronize()
    a, b = g.cpu().numpy(), g2.cpu().numpy()
    assert rel_l2(a, oracle.reward_scan(c.astype(np.float64), 1000, 0.95)) <= 1e-5
    changed = np.nonzero((a != b).any(0))[0]
    assert changed.min() >= 1000 and changed.max() <= 1500


@pytest.mark.parametrize("K,T,N,L,gamma", [(16, 256, 512, 128, 0.0), (9, 60, 100, 20, 0.7),
                                           (70, 12, 4096, 12, 0.0), (5, 6, 8192, 3, 0.9),
                                           (3, 4, 40000, 4, 0.0), (2, 3, 4, 1, 0.0),
                                           (3, 2, 65536, 2, 0.5)])  # N = DUST_N_MAX: 16 waves
def test_error_estimate(K, T, N, L, gamma):
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(N)
    c = rng.standard_normal((K, T)) * 0.03
    r = oracle.reward_scan(c, L, gamma)
    sigma, seed, stream = 0.02, 77, 4
    g = dust.error_estimate(_cuda(torch.from_numpy(r.astype(np.float32))), N=N, sigma=sigma,
                            seed=seed, stream=stream)
    torch.cuda.synchronize()
    ref = oracle.linear_rows(c, L, N, sigma, gamma, seed, list(range(T)), stream)
    assert_parity(g.cpu().numpy(), ref, "g_hat")


@pytest.mark.parametrize("T,N,d,bf16", [(600, 1000, 72, True), (600, 1000, 72, False),
                                         (1, 5, 3, False), (4097, 300, 129, True),
                                         (2048, 512, 512, True), (31, 64, 64, False),
                                         # several token splits, ragged last split,
                                         # N % 4 != 0, three column tiles
                                         (9000, 257, 520, True), (20000, 384, 256, False),
                                         (16417, 129, 264, True), (130, 4100, 8, True)])
def test_outer_sum(T, N, d, bf16):
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(T * 7 + d)
    g = rng.standard_normal((T, N)).astype(np.float32)
    Xf = rng.standard_normal((T, d)).astype(np.float32)
    X = torch.from_numpy(Xf).to(torch.bfloat16) if bf16 else torch.from_numpy(Xf)
    G = dust.outer_sum(_cuda(torch.from_numpy(g)), _cuda(X))
    torch.cuda.synchronize()
    ref = oracle.outer_sum(g.astype(np.float64), synth.to_f64(X))
    assert_parity(G.cpu().numpy(), ref, "G_W")
    # relative to each entry's scale sum_t |g||x| the error stays near fp32 level
    scale = np.abs(g.astype(np.float64)).T @ np.abs(synth.to_f64(X))
    assert (np.abs(G.cpu().numpy() - ref) <= 2e-5 * scale + 1e-30).all()


def test_check_targets():
    dust = need_gpu()
    import torch
    y = torch.randint(0, 100, (1000,), dtype=torch.int32, device="cuda")
    assert dust.check_targets(y, 100)
    y[517] = 100
    assert not dust.check_targets(y, 100)
    y[517] = -1
    assert not dust.check_targets(y, 100)


def test_reward_scan_more_jobs_than_grid():
    """K * T / L = 524288 (draw, sequence) jobs: more than the scan's grid of
    65536 workgroups x 4 waves, so every wave walks several jobs."""
    dust = need_gpu()
    import torch
    K, T, L = 4096, 256, 2
    c = np.random.default_rng(11).standard_normal((K, T)).astype(np.float32)
    r = dust.reward_scan(_cuda(torch.from_numpy(c)), seq_len=L, gamma=0.75)
    torch.cuda.synchronize()
    ref = oracle.reward_scan(c.astype(np.float64), L, 0.75)
    assert rel_l2(r.cpu().numpy(), ref) <= 1e-5


def test_outer_sum_planes_grid_stride():
    """fp32 X with T * d / 8 above the plane pass's 16384 x 256 threads, so the
    pass strides; d = 520 also leaves a ragged column tile."""
    dust = need_gpu()
    import torch
    T, N, d = 65536, 32, 520
    rng = np.random.default_rng(5)
    g = rng.standard_normal((T, N)).astype(np.float32)
    Xf = rng.standard_normal((T, d)).astype(np.float32)
    G = dust.outer_sum(_cuda(torch.from_numpy(g)), _cuda(torch.from_numpy(Xf)))
    torch.cuda.synchronize()
    ref = oracle.outer_sum(g.astype(np.float64), Xf.astype(np.float64))
    assert_parity(G.cpu().numpy(), ref, "G_W")
