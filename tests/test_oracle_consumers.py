"""Pins of the oracle's consumers of the estimate (no GPU): the embedding
scatter-add against the outer product with one-hot inputs (the identity the
paper digest states in section 2.2) and against numpy's add.at; the optimiser
steps against torch.optim (an independent implementation) in fp64; the
closed-form head gradient against torch autograd of cross_entropy."""
import numpy as np
import torch

import oracle


def test_embedding_is_outer_product_with_one_hot():
    rng = np.random.default_rng(0)
    T, N, vocab = 50, 12, 9
    ids = rng.integers(-1, vocab + 1, T).astype(np.int32)  # includes out-of-range ids
    g = rng.standard_normal((T, N))
    GE = oracle.embedding_grad(ids, g, vocab)
    onehot = np.zeros((T, vocab))
    ok = (ids >= 0) & (ids < vocab)
    onehot[np.arange(T)[ok], ids[ok]] = 1.0
    np.testing.assert_allclose(GE, oracle.outer_sum(g, onehot).T, rtol=1e-12, atol=1e-12)
    ref = np.zeros((vocab, N))
    np.add.at(ref, ids[ok], g[ok])
    np.testing.assert_allclose(GE, ref, rtol=1e-12, atol=1e-12)


def test_sgd_momentum_matches_torch():
    rng = np.random.default_rng(1)
    W0 = rng.standard_normal(40)
    Gs = [rng.standard_normal(40) for _ in range(3)]
    w = torch.tensor(W0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.SGD([w], lr=0.05, momentum=0.9, weight_decay=0.01)
    W, m = W0.copy(), np.zeros(40)
    for G in Gs:
        w.grad = torch.tensor(G, dtype=torch.float64)
        opt.step()
        W, m = oracle.sgd_momentum(W, G, m, 0.05, 0.9, 0.01)
    np.testing.assert_allclose(W, w.detach().numpy(), rtol=1e-12, atol=1e-14)


def test_adam_matches_torch():
    rng = np.random.default_rng(2)
    W0 = rng.standard_normal(40)
    Gs = [rng.standard_normal(40) for _ in range(4)]
    w = torch.tensor(W0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([w], lr=0.01, betas=(0.9, 0.99), eps=1e-6, weight_decay=0.02)
    W, m, v = W0.copy(), np.zeros(40), np.zeros(40)
    for k, G in enumerate(Gs, start=1):
        w.grad = torch.tensor(G, dtype=torch.float64)
        opt.step()
        W, m, v = oracle.adam(W, G, m, v, 0.01, k, 0.9, 0.99, 1e-6, 0.02)
    np.testing.assert_allclose(W, w.detach().numpy(), rtol=1e-12, atol=1e-14)


def test_ce_grad_matches_autograd():
    rng = np.random.default_rng(3)
    z = torch.tensor(rng.standard_normal((7, 33)) * 2, dtype=torch.float64, requires_grad=True)
    y = torch.tensor(rng.integers(0, 33, 7))
    torch.nn.functional.cross_entropy(z, y, reduction="sum").backward()
    np.testing.assert_allclose(oracle.ce_grad(z.detach().numpy(), y.numpy()), z.grad.numpy(),
                               rtol=1e-12, atol=1e-14)
