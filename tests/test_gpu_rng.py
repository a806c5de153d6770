"""GPU noise stage against the oracle: raw Philox bit-exact, normals within the
fp32 transcendental error (|error| <= 1e-5: v_log/v_sqrt/v_sin/v_cos are good to
a few ulp, and |a| <= 5.77)."""
import numpy as np
import pytest

import oracle
from util import need_gpu

pytestmark = pytest.mark.gpu

NOISE_ABS = 1e-5


@pytest.mark.parametrize("seed", [0, 1, 0xFFFFFFFF, 0x123456789ABCDEF0, 2**64 - 1])
def test_philox_raw_bit_exact(seed):
    dust = need_gpu()
    import torch
    rng = np.random.default_rng(seed & 0xFFFF)
    ctr = rng.integers(0, 2**32, size=(300_000, 4), dtype=np.uint64).astype(np.uint32)
    edges = np.array([0, 1, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFF], dtype=np.uint32)
    e = np.array(np.meshgrid(edges, edges, edges, edges)).T.reshape(-1, 4)
    ctr = np.ascontiguousarray(np.concatenate([e, ctr]))
    out = dust.philox4x32_10(seed, torch.from_numpy(ctr.view(np.int32)).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.philox4x32_10(seed, ctr))


def test_philox_empty():
    dust = need_gpu()
    import torch
    out = dust.philox4x32_10(3, torch.empty((0, 4), dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 4)


@pytest.mark.parametrize("shape", [(3, 37, 100, 0, 0), (2, 5, 4, 7, 3), (1, 64, 4096, 1, 0),
                                   (4, 3, 8192, 60, 5)])
def test_noise_matches_oracle(shape):
    dust = need_gpu()
    import torch
    ndraw, T, N, draw0, stream = shape
    seed = 0xABCDEF12345
    a = dust.noise(seed=seed, stream=stream, draw0=draw0, ndraw=ndraw, T=T, N=N)
    torch.cuda.synchronize()
    ref = oracle.noise(seed, stream, draw0, ndraw, T, N)
    err = np.abs(a.cpu().numpy().astype(np.float64) - ref)
    assert err.max() <= NOISE_ABS, err.max()


def test_noise_large_grid_statistics():
    # A grid larger than one launch wave (grid-stride loop): standard normal.
    dust = need_gpu()
    import torch
    a = dust.noise(seed=11, stream=0, ndraw=8, T=4096, N=2048)
    x = a.double()
    n = x.numel()
    assert abs(x.mean().item()) < 5 / np.sqrt(n)
    assert abs(x.var().item() - 1) < 5 * np.sqrt(2 / n)
    # spot rows against the oracle
    ref = oracle.noise(11, 0, 7, 1, 4096, 2048)[0]
    assert np.abs(a[7].cpu().numpy() - ref).max() <= NOISE_ABS
