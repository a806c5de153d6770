"""Pins of the oracle's noise stream (no GPU).

The pages fix only that the noise is standard normal and independent per token
and draw (laoyaoba analysis, mechanism section; linlog explainer, "the core of
Dust").  The oracle realises it as Philox4x32-10 (Salmon et al., SC'11) +
Box-Muller (1958).  Pinned here against things other than the oracle itself:
  - the raw Philox stream against two independent open-source implementations
    compiled on this host (ATen's PhiloxRNGEngine, rocRAND's philox4x32_10),
  - the uniform (radius) and angle maps by exact integer arithmetic,
  - Box-Muller by inverting it (radius and angle give back the uniforms) and by
    the distribution (moments, Kolmogorov-Smirnov against scipy's normal),
    with neighbouring coordinates uncorrelated.
"""
import ctypes
import os

import numpy as np
import pytest
import scipy.stats

import oracle
from util import pin_lib

TORCH_INC = None


def _torch_include():
    import torch
    return os.path.join(os.path.dirname(torch.__file__), "include")


def _edge_counters(rng, n):
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    edges = np.array([0, 1, 2, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFE, 0xFFFFFFFF], dtype=np.uint32)
    e = np.array(np.meshgrid(edges, edges, edges[:3], edges[:3])).T.reshape(-1, 4)
    return np.ascontiguousarray(np.concatenate([e, ctr]).astype(np.uint32))


def _call(lib, fn, seed, ctr):
    out = np.empty_like(ctr)
    f = getattr(lib, fn)
    f.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    f.restype = None
    f(seed, ctr.ctypes.data, out.ctypes.data, ctr.shape[0])
    return out


SEEDS = [0, 1, 0xFFFFFFFF, 0x100000000, 0x123456789ABCDEF0, 2**64 - 1]


@pytest.mark.parametrize("seed", SEEDS)
def test_philox_matches_aten(seed):
    lib = pin_lib("philox_aten", ["g++"], ["-I", _torch_include()])
    rng = np.random.default_rng(seed & 0xFFFF)
    ctr = _edge_counters(rng, 200_000)
    assert np.array_equal(oracle.philox4x32_10(seed, ctr), _call(lib, "aten_philox_batch", seed, ctr))


@pytest.mark.parametrize("seed", SEEDS)
def test_philox_matches_rocrand(seed):
    lib = pin_lib("philox_rocrand", ["hipcc"], [])
    rng = np.random.default_rng(seed & 0xFFFF)
    ctr = _edge_counters(rng, 200_000)
    ctr[:, 1] &= (1 << 30) - 1  # rocRAND's offset is counted in words (see the pin source)
    assert np.array_equal(oracle.philox4x32_10(seed, ctr),
                          _call(lib, "rocrand_philox_batch", seed, ctr))


def test_philox_distinct_counters_distinct_blocks():
    # Philox is a bijection of the counter for a fixed key: no two of these collide.
    rng = np.random.default_rng(3)
    ctr = np.unique(rng.integers(0, 2**32, size=(50_000, 4), dtype=np.uint64).astype(np.uint32), axis=0)
    out = oracle.philox4x32_10(7, ctr)
    assert np.unique(out, axis=0).shape[0] == ctr.shape[0]


def test_uniform_map_exact():
    x = np.array([0, 1, 511, 512, 0x7FFFFFFF, 0x80000000, 0xFFFFFE00, 0xFFFFFFFF], dtype=np.uint32)
    x = np.concatenate([x, np.random.default_rng(1).integers(0, 2**32, 100_000, dtype=np.uint64).astype(np.uint32)])
    u = oracle.uniform(x)
    m = (u - 2.0**-24) * 2.0**23
    assert np.array_equal(m, np.floor(m))                      # an integer ...
    assert np.array_equal(m.astype(np.int64), (x >> 9).astype(np.int64))  # ... equal to the top 23 bits
    assert (u > 0).all() and (u < 1).all()
    assert u.min() == 2.0**-24 and u[x == 0xFFFFFFFF][0] == 1 - 2.0**-24
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)  # exact in fp32


def test_angle_map_exact():
    # v = m / 2^23 with m the top 23 bits: [0, 1) revolutions, 0 included
    x = np.array([0, 1, 511, 512, 0x7FFFFFFF, 0x80000000, 0xFFFFFE00, 0xFFFFFFFF], dtype=np.uint32)
    x = np.concatenate([x, np.random.default_rng(2).integers(0, 2**32, 100_000, dtype=np.uint64).astype(np.uint32)])
    v = oracle.angle(x)
    m = v * 2.0**23
    assert np.array_equal(m, np.floor(m))
    assert np.array_equal(m.astype(np.int64), (x >> 9).astype(np.int64))
    assert (v >= 0).all() and (v < 1).all()
    assert v[x == 511][0] == 0 and v[x == 512][0] == 2.0**-23
    assert v[x == 0xFFFFFFFF][0] == 1 - 2.0**-23
    assert np.array_equal(v.astype(np.float32).astype(np.float64), v)  # exact in fp32
    # the radius uniform of the same word is the angle plus half a step
    assert np.array_equal(oracle.uniform(x), v + 2.0**-24)


def test_box_muller_inverts_to_the_block_uniforms():
    # a[4j]^2 + a[4j+1]^2 = -2 ln u0 and atan2(a[4j+1], a[4j]) = 2 pi v1 (mod 2 pi),
    # u0 the uniform of word 0 and v1 the angle of word 1; likewise columns
    # 4j+2, 4j+3 with words 2 and 3.  This fixes which Philox word feeds which
    # column and which map each word goes through.
    seed, stream, T, N, ndraw = 5, 3, 7, 64, 3
    a = oracle.noise(seed, stream, 0, ndraw, T, N)
    for i in range(ndraw):
        for t in range(T):
            ctr = np.array([[t, j, i, stream] for j in range(N // 4)], dtype=np.uint32)
            words = oracle.philox4x32_10(seed, ctr).ravel()
            u = oracle.uniform(words).reshape(-1, 4)
            v = oracle.angle(words).reshape(-1, 4)
            row = a[i, t].reshape(-1, 4)
            for p in (0, 1):
                c, s = row[:, 2 * p], row[:, 2 * p + 1]
                np.testing.assert_allclose(c * c + s * s, -2 * np.log(u[:, 2 * p]), rtol=1e-12)
                ang = np.mod(np.arctan2(s, c) / (2 * np.pi), 1.0)
                d = np.abs(ang - v[:, 2 * p + 1])
                assert np.minimum(d, 1 - d).max() < 1e-12
                # half a step of 2^-23 off: the uniform map in the angle is caught
                d_u = np.abs(ang - u[:, 2 * p + 1])
                assert np.minimum(d_u, 1 - d_u).min() > 2.0**-25


def test_noise_draw_offset():
    # out[k] is draw draw0 + k
    a = oracle.noise(9, 0, 0, 6, 5, 16)
    b = oracle.noise(9, 0, 4, 2, 5, 16)
    assert np.array_equal(a[4:6], b)


def test_noise_is_standard_normal():
    a = oracle.noise(1, 0, 0, 4, 1024, 2560).ravel()  # 1.05e7 samples
    n = a.size
    assert abs(a.mean()) < 5 / np.sqrt(n)
    assert abs(a.var() - 1) < 5 * np.sqrt(2 / n)
    assert abs(scipy.stats.kurtosis(a, fisher=False) - 3) < 5 * np.sqrt(24 / n)
    assert abs(scipy.stats.skew(a)) < 5 * np.sqrt(6 / n)
    ks = scipy.stats.kstest(a, "norm")
    assert ks.pvalue > 1e-4, ks
    assert np.abs(a).max() <= np.sqrt(48 * np.log(2)) + 1e-12  # u >= 2^-24 caps the tails


def test_noise_coordinates_uncorrelated():
    a = oracle.noise(2, 0, 0, 8, 256, 512)  # [draw, token, column]
    n = a[:, :, :-1].size
    for x, y in ((a[:, :, :-1], a[:, :, 1:]),      # neighbouring columns (same and next block)
                 (a[:, :, 0::4], a[:, :, 1::4]),   # the two outputs of one Box-Muller pair
                 (a[:, :-1], a[:, 1:]),            # neighbouring tokens
                 (a[:-1], a[1:])):                 # neighbouring draws
        r = np.corrcoef(x.ravel(), y.ravel())[0, 1]
        assert abs(r) < 6 / np.sqrt(min(n, x.size)), r
    # a different stream word gives an unrelated stream
    b = oracle.noise(2, 1, 0, 8, 256, 512)
    assert abs(np.corrcoef(a.ravel(), b.ravel())[0, 1]) < 6 / np.sqrt(a.size)
