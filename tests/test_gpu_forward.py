"""The perturbed forward of a hidden linear layer, Y[k] = X W^T + sigma a^(draw0+k)
(paper digest, sections 2 and 2.1), against the oracle; and its agreement with
dust_linear_estimate: for a loss linear in y, L_t = u_t . y_t, the estimator fed
with the centred decreases of the forward's own perturbed outputs converges to
u_t (its cosine follows the same law as the head's, (1-1/K)/sqrt((1-1/K)^2 +
(N+1)/K)).  Tolerance: relative L2 1e-5 on Y (fp32 accumulation of exact bf16
products; fp32 operands split into bf16 hi + lo)."""
import numpy as np
import pytest

import oracle
from activation_perturbation_estimator_amd import synth
from util import need_gpu, rel_l2

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,d,N,ndraw,bf16", [(300, 72, 200, 3, True), (300, 72, 200, 3, False),
                                               (128, 512, 2048, 1, True), (5, 8, 4, 2, False),
                                               (257, 136, 132, 2, True)])
def test_perturbed_linear_matches_oracle(T, d, N, ndraw, bf16):
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(T + d + N)
    Xf = rng.standard_normal((T, d)).astype(np.float32) / np.sqrt(d)
    Wf = rng.standard_normal((N, d)).astype(np.float32) / np.sqrt(d)
    dt = torch.bfloat16 if bf16 else torch.float32
    X = torch.from_numpy(Xf).to(dt)
    W = torch.from_numpy(Wf).to(dt)
    sigma, seed, stream, draw0 = 0.05, 77, 2, 5
    Y = dust.perturbed_linear(X.cuda(), W.cuda(), sigma=sigma, seed=seed, stream=stream,
                              draw0=draw0, ndraw=ndraw)
    torch.cuda.synchronize()
    ref = oracle.perturbed_linear(synth.to_f64(X), synth.to_f64(W), sigma, seed, stream, draw0,
                                  ndraw)
    got = Y.cpu().numpy()
    assert rel_l2(got, ref) <= 1e-5, rel_l2(got, ref)
    assert np.abs(got - ref).max() <= 1e-4


def test_forward_and_estimate_share_the_noise():
    dust = need_gpu()
    import torch
    T, d, N, K, sigma, seed = 64, 32, 96, 4096, 0.01, 9
    rng = np.random.default_rng(3)
    X = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).cuda()
    W = torch.from_numpy(rng.standard_normal((N, d)).astype(np.float32)).cuda()
    u = torch.from_numpy(rng.standard_normal((T, N)).astype(np.float32)).cuda()
    losses = torch.empty((K, T), dtype=torch.float64, device="cuda")
    for k0 in range(0, K, 512):
        Y = dust.perturbed_linear(X, W, sigma=sigma, seed=seed, draw0=k0, ndraw=512)
        losses[k0:k0 + 512] = (Y.double() * u.double()[None]).sum(-1)
    dec = -losses                                  # loss decrease up to a per-token constant
    c = (dec - dec.mean(0, keepdim=True)).float().contiguous()
    g, _ = dust.linear_estimate(X, c, N=N, sigma=sigma, gamma=0.0, seed=seed, seq_len=T)
    torch.cuda.synchronize()
    g = g.double().cpu().numpy()
    uu = u.double().cpu().numpy()
    cos = (g * uu).sum(1) / np.linalg.norm(g, axis=1) / np.linalg.norm(uu, axis=1)
    k = 1 - 1 / K
    pred = k / np.sqrt(k * k + (N + 1) / K)
    assert abs(cos.mean() - pred) < 3 * cos.std() / np.sqrt(T) + 0.01, (cos.mean(), pred)
    beta = (g * uu).sum(1) / (uu * uu).sum(1)
    assert abs(beta.mean() - k) < 4 * np.sqrt(2.0 / K) / np.sqrt(T) + 0.01, beta.mean()
