"""The Python binding refuses tensors whose shape, dtype or device does not
match what the C ABI will read or write (the ABI takes bare pointers, so a
short output buffer would otherwise be overrun).  These checks run before any
GPU work, so CPU tensors exercise them here."""
import pytest
import torch

import activation_perturbation_estimator_amd as dust


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def test_head_estimate_checks_inputs_and_outputs():
    z, y, X = f32(8, 16), i32(8), f32(8, 4)
    with pytest.raises(ValueError, match="targets must have shape"):
        dust.head_estimate(z, i32(7), X, sigma=0.1, K=2)
    with pytest.raises(TypeError, match="targets must be"):
        dust.head_estimate(z, y.long(), X, sigma=0.1, K=2)
    with pytest.raises(ValueError, match="X must have shape"):
        dust.head_estimate(z, y, f32(9, 4), sigma=0.1, K=2)
    with pytest.raises(TypeError, match="logits must be"):
        dust.head_estimate(z.double(), y, X, sigma=0.1, K=2)
    with pytest.raises(ValueError, match="G_W must have shape"):
        dust.head_estimate(z, y, X, sigma=0.1, K=2, out=(f32(8, 16), f32(16, 3)))
    with pytest.raises(TypeError, match="g_hat must be"):
        dust.head_estimate(z, y, X, sigma=0.1, K=2,
                           out=(torch.zeros(8, 16, dtype=torch.bfloat16), f32(16, 4)))
    with pytest.raises(ValueError, match="out must hold 2"):
        dust.head_estimate(z, y, X, sigma=0.1, K=2, out=(f32(8, 16),))
    # shapes right: only then the device check
    with pytest.raises(ValueError, match="GPU tensor"):
        dust.head_estimate(z, y, X, sigma=0.1, K=2, out=(f32(8, 16), f32(16, 4)))


def test_linear_and_stage_outputs():
    X, c = f32(8, 4), f32(3, 8)
    with pytest.raises(ValueError, match="c must have shape"):
        dust.linear_estimate(X, f32(3, 9), N=12, sigma=0.1)
    with pytest.raises(ValueError, match="g_hat must have shape"):
        dust.linear_estimate(X, c, N=12, sigma=0.1, out=(f32(8, 8), f32(12, 4)))
    with pytest.raises(ValueError, match="out must have shape"):
        dust.error_estimate(c, N=12, sigma=0.1, out=f32(8, 8))
    with pytest.raises(TypeError, match="r must be"):
        dust.error_estimate(c.double(), N=12, sigma=0.1)
    with pytest.raises(ValueError, match="out must have shape"):
        dust.centre(c, out=f32(3, 7))
    with pytest.raises(ValueError, match="out must have shape"):
        dust.reward_scan(c, seq_len=4, gamma=0.5, out=f32(2, 8))
    with pytest.raises(ValueError, match="X must have shape"):
        dust.outer_sum(f32(8, 12), f32(7, 4))
    with pytest.raises(ValueError, match="out must have shape"):
        dust.outer_sum(f32(8, 12), f32(8, 4), out=f32(4, 12))


def test_consumer_checks():
    with pytest.raises(ValueError, match="W must have shape"):
        dust.perturbed_linear(f32(8, 16), f32(12, 8), sigma=0.1)
    with pytest.raises(TypeError, match="W must be"):
        dust.perturbed_linear(f32(8, 16), torch.zeros(12, 16, dtype=torch.bfloat16), sigma=0.1)
    with pytest.raises(ValueError, match="out must have shape"):
        dust.perturbed_linear(f32(8, 16), f32(12, 16), sigma=0.1, ndraw=2, out=f32(1, 8, 12))
    with pytest.raises(ValueError, match="ids must have shape"):
        dust.embedding_grad(i32(7), f32(8, 4), 10)
    with pytest.raises(ValueError, match="out must have shape"):
        dust.embedding_grad(i32(8), f32(8, 4), 10, out=f32(9, 4))
    with pytest.raises(ValueError, match="G must have shape"):
        dust.sgd_momentum_(f32(10), f32(9), f32(10), lr=0.1)
    with pytest.raises(TypeError, match="v must be"):
        dust.adam_(f32(10), f32(10), f32(10), torch.zeros(10, dtype=torch.float64), lr=0.1, step=1)
    with pytest.raises(ValueError, match="out must have shape"):
        dust.ce_grad(f32(4, 8), i32(4), out=f32(4, 7))
    with pytest.raises(ValueError, match="ctr must be"):
        dust.philox4x32_10(1, torch.zeros(5, 4, dtype=torch.int64))
