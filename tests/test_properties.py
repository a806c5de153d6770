"""Property-based checks on the CPU (hypothesis).

Oracle invariants that hold for every input, whatever its shape or values:
  - centring (paper digest, section 2.2: the centred loss decrease): the
    centred values of one token sum to zero over its draws, and centring does
    not see the clean loss;
  - the discounted reward (same section): r_t - gamma r_{t+1} = c_t inside a
    sequence, r = c at a sequence's last token, and sequences do not see each
    other;
  - the error estimate is linear in the rewards: g(c1 + s c2) = g(c1) + s g(c2)
    with the same noise, and G_W = g^T X.
The C ABI's host-side checks over random argument tuples: no call crashes, and
each answer follows from the rules include/dust.h states (a null pointer, a bad
enum, size or parameter is DUST_ERR_INVALID_ARG; a size beyond the limits with
valid arguments is DUST_ERR_UNSUPPORTED; a short workspace is
DUST_ERR_WORKSPACE; a call that passes every check reaches HIP, which on this
GPU-less machine fails with DUST_ERR_HIP).  These ABI checks stay off any
machine with a GPU, where a call that passes its checks would launch kernels
on the fake pointers they use.
"""
import math

import numpy as np
import pytest
from hypothesis import HealthCheck, assume, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])
ABI_SETTINGS = settings(max_examples=400, deadline=None,
                        suppress_health_check=[HealthCheck.too_slow])


# --------------------------------------------------------------------------
# Oracle invariants
# --------------------------------------------------------------------------

@SETTINGS
@given(K=st.integers(1, 9), nseq=st.integers(1, 3), L=st.integers(1, 6),
       V=st.sampled_from([4, 8, 12]), sigma=st.floats(1e-3, 1.0),
       gamma=st.sampled_from([0.0, 0.5, 1.0]), seed=st.integers(0, 2**64 - 1),
       data_seed=st.integers(0, 2**31 - 1))
def test_centred_values_sum_to_zero_per_token(K, nseq, L, V, sigma, gamma, seed, data_seed):
    rng = np.random.default_rng(data_seed)
    T = nseq * L
    z = rng.normal(0.0, 2.0, (T, V))
    y = rng.integers(0, V, T)
    X = rng.normal(0.0, 1.0, (T, 3))
    _, _, diag = oracle.head_estimate(z, y, X, L, sigma, K, gamma, seed, diagnostics=True)
    c = diag["c"]
    scale = np.abs(c).sum(axis=0) + 1e-300
    assert np.all(np.abs(c.sum(axis=0)) <= 1e-12 * scale + 1e-300)
    # c = mean over draws of the losses minus the draw's loss: the clean loss cancels
    ell = diag["ell"]
    np.testing.assert_allclose(c, ell.mean(axis=0)[None, :] - ell, rtol=0, atol=1e-12)


@SETTINGS
@given(K=st.integers(1, 5), nseq=st.integers(1, 4), L=st.integers(1, 40),
       gamma=st.floats(0.0, 1.0), data_seed=st.integers(0, 2**31 - 1))
def test_reward_recurrence_and_sequence_isolation(K, nseq, L, gamma, data_seed):
    rng = np.random.default_rng(data_seed)
    T = nseq * L
    c = rng.normal(0.0, 1.0, (K, T))
    r = oracle.reward_scan(c, L, gamma)
    for q in range(nseq):
        seg = slice(q * L, (q + 1) * L)
        rs, cs = r[:, seg], c[:, seg]
        np.testing.assert_array_equal(rs[:, -1], cs[:, -1])
        lhs = rs[:, :-1] - gamma * rs[:, 1:]
        np.testing.assert_allclose(lhs, cs[:, :-1], rtol=0,
                                   atol=1e-12 * (1 + np.abs(rs).max()))
    # changing one sequence's c leaves every other sequence's r as it was
    if nseq > 1:
        c2 = c.copy()
        c2[:, :L] += rng.normal(0.0, 1.0, (K, L))
        r2 = oracle.reward_scan(c2, L, gamma)
        np.testing.assert_array_equal(r2[:, L:], r[:, L:])


@SETTINGS
@given(K=st.integers(1, 6), L=st.integers(1, 5), nseq=st.integers(1, 3),
       N=st.sampled_from([4, 8, 16]), d=st.integers(1, 5), sigma=st.floats(1e-3, 2.0),
       gamma=st.floats(0.0, 1.0), s=st.floats(-3.0, 3.0), seed=st.integers(0, 2**64 - 1),
       data_seed=st.integers(0, 2**31 - 1))
def test_error_estimate_is_linear_in_the_rewards(K, L, nseq, N, d, sigma, gamma, s, seed,
                                                 data_seed):
    rng = np.random.default_rng(data_seed)
    T = nseq * L
    X = rng.normal(0.0, 1.0, (T, d))
    c1 = rng.normal(0.0, 1.0, (K, T))
    c2 = rng.normal(0.0, 1.0, (K, T))
    g1, G1 = oracle.linear_estimate(X, c1, L, N, sigma, gamma, seed)
    g2, G2 = oracle.linear_estimate(X, c2, L, N, sigma, gamma, seed)
    g, G = oracle.linear_estimate(X, c1 + s * c2, L, N, sigma, gamma, seed)
    tol = 1e-10 * (np.abs(g1).max() + abs(s) * np.abs(g2).max() + 1e-300)
    np.testing.assert_allclose(g, g1 + s * g2, rtol=0, atol=tol)
    np.testing.assert_allclose(G, g.T @ X, rtol=1e-12, atol=1e-12 * np.abs(G).max())


# --------------------------------------------------------------------------
# C ABI host-side checks
# --------------------------------------------------------------------------

FAKE = 0x1000  # never dereferenced: every such call is rejected or fails in HIP first


def _abi():
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("random ABI arguments are only sent where no GPU can run them")
    except ImportError:
        pass
    from activation_perturbation_estimator_amd import _lib as L
    return L, L.load()


I64 = st.one_of(st.integers(-2**63, 2**63 - 1), st.integers(-8, 70000),
                st.sampled_from([0, 1, 4, 8, 2**20, 2**22, 2**22 + 1, 2**24, 2**31, 2**32,
                                 2**40, 2**62, 2**63 - 1, -2**63]))
F32 = st.one_of(st.floats(allow_nan=True, allow_infinity=True, width=32),
                st.sampled_from([0.0, 0.01, 0.5, 1.0, 8.0, 8.5, -0.0]))
ENUM = st.one_of(st.sampled_from([0, 1]), st.integers(-2**31, 2**31 - 1))
PTR = st.sampled_from([None, FAKE])

HIP_FAIL = 3  # DUST_ERR_HIP
SIGMA_MAX = 8.0
N_MAX = 65536
T_MAX = 2**22
WIDTH_MAX = 2**20
K_MAX = 2**31 - 64
ELEMS_MAX = 2**40


def _sigma_ok(x):
    return math.isfinite(x) and 0.0 < x <= SIGMA_MAX


def _gamma_ok(x):
    return math.isfinite(x) and 0.0 <= x <= 1.0


def _f32(x):
    return float(np.float32(x))


@ABI_SETTINGS
@given(logits=PTR, targets=PTR, X=PTR, g=PTR, G=PTR, zdt=ENUM, xdt=ENUM, T=I64, V=I64, d=I64,
       L=I64, sigma=F32, K=I64, gamma=F32, ws=PTR, wsb=st.integers(0, 2**62))
def test_head_estimate_answers_by_its_rules(logits, targets, X, g, G, zdt, xdt, T, V, d, L,
                                            sigma, K, gamma, ws, wsb):
    Lb, lib = _abi()
    sigma, gamma = _f32(sigma), _f32(gamma)
    st_ = lib.dust_head_estimate(logits, zdt, targets, X, xdt, T, V, d, L, sigma, K, gamma,
                                 1, 0, g, G, None, ws, wsb, None, None)
    invalid = (None in (logits, targets, X, g, G) or zdt not in (0, 1) or xdt not in (0, 1)
               or T <= 0 or V <= 0 or V % 4 != 0 or V > N_MAX or d <= 0 or K <= 0
               or K > K_MAX or L <= 0 or (T > 0 and L > 0 and T % L != 0)
               or not _sigma_ok(sigma) or not _gamma_ok(gamma))
    beyond = (T > T_MAX or d > WIDTH_MAX)
    if invalid:
        assert st_ in (Lb.DUST_ERR_INVALID_ARG, Lb.DUST_ERR_UNSUPPORTED)
        if not beyond:
            assert st_ == Lb.DUST_ERR_INVALID_ARG
        return
    if beyond:
        assert st_ == Lb.DUST_ERR_UNSUPPORTED
        return
    assert st_ in (Lb.DUST_ERR_UNSUPPORTED, Lb.DUST_ERR_WORKSPACE, HIP_FAIL)
    need = lib.dust_head_workspace_size(T, V, d, K, gamma)
    assert need >= 256
    if st_ != Lb.DUST_ERR_UNSUPPORTED:
        assert (st_ == Lb.DUST_ERR_WORKSPACE) == (ws is None or wsb < need)


@ABI_SETTINGS
@given(X=PTR, c=PTR, g=PTR, G=PTR, xdt=ENUM, T=I64, d=I64, N=I64, L=I64, sigma=F32, K=I64,
       gamma=F32, draw0=I64, K_total=I64, ws=PTR, wsb=st.integers(0, 2**62))
def test_linear_estimate_answers_by_its_rules(X, c, g, G, xdt, T, d, N, L, sigma, K, gamma,
                                              draw0, K_total, ws, wsb):
    Lb, lib = _abi()
    sigma, gamma = _f32(sigma), _f32(gamma)
    st_ = lib.dust_linear_estimate(X, xdt, c, T, d, N, L, sigma, K, gamma, 1, 0, draw0, K_total,
                                   g, G, ws, wsb, None, None)
    draws_bad = (draw0 < 0 or K_total < 1 or K_total > K_MAX
                 or (K > 0 and draw0 > 2**32 - K))
    invalid = (None in (X, c, g, G) or xdt not in (0, 1) or draws_bad or T <= 0 or N <= 0
               or N % 4 != 0 or N > N_MAX or d <= 0 or K <= 0 or K > K_MAX or L <= 0
               or (T > 0 and L > 0 and T % L != 0) or not _sigma_ok(sigma)
               or not _gamma_ok(gamma))
    beyond = (T > T_MAX or d > WIDTH_MAX)
    if invalid:
        assert st_ in (Lb.DUST_ERR_INVALID_ARG, Lb.DUST_ERR_UNSUPPORTED)
        if not beyond:
            assert st_ == Lb.DUST_ERR_INVALID_ARG
        return
    if beyond:
        assert st_ == Lb.DUST_ERR_UNSUPPORTED
        return
    assert st_ in (Lb.DUST_ERR_UNSUPPORTED, Lb.DUST_ERR_WORKSPACE, HIP_FAIL)
    need = lib.dust_linear_workspace_size(T, d, N, K, gamma)
    assert need >= 256
    if st_ != Lb.DUST_ERR_UNSUPPORTED:
        assert (st_ == Lb.DUST_ERR_WORKSPACE) == (ws is None or wsb < need)


@ABI_SETTINGS
@given(r=PTR, g=PTR, K=I64, T=I64, N=I64, sigma=F32, draw0=I64, K_total=I64)
def test_error_estimate_answers_by_its_rules(r, g, K, T, N, sigma, draw0, K_total):
    Lb, lib = _abi()
    sigma = _f32(sigma)
    st_ = lib.dust_error_estimate(r, K, T, N, sigma, 1, 0, draw0, K_total, g, None)
    invalid = (None in (r, g) or K <= 0 or K > K_MAX or T <= 0 or N <= 0 or N % 4 != 0
               or N > N_MAX or not _sigma_ok(sigma) or draw0 < 0 or K_total < 1
               or K_total > K_MAX or (K > 0 and draw0 > 2**32 - K))
    if invalid:
        assert st_ == Lb.DUST_ERR_INVALID_ARG
    elif T >= 2**24 or T * N > ELEMS_MAX or K * T > ELEMS_MAX:
        assert st_ == Lb.DUST_ERR_UNSUPPORTED
    else:
        assert st_ == HIP_FAIL


@ABI_SETTINGS
@given(out=PTR, draw0=I64, ndraw=I64, T=I64, N=I64)
def test_noise_answers_by_its_rules(out, draw0, ndraw, T, N):
    Lb, lib = _abi()
    st_ = lib.dust_noise(1, 0, draw0, ndraw, T, N, out, None)
    invalid = (out is None or ndraw < 0 or T < 0 or N <= 0 or N % 4 != 0 or N > N_MAX
               or draw0 < 0 or (ndraw >= 0 and draw0 > 2**32 - ndraw) or T > 2**32)
    if invalid:
        assert st_ == Lb.DUST_ERR_INVALID_ARG
    elif ndraw * T > ELEMS_MAX // N:
        assert st_ == Lb.DUST_ERR_UNSUPPORTED
    else:
        assert st_ in (Lb.DUST_OK, HIP_FAIL)  # nothing to do when ndraw * T == 0


@ABI_SETTINGS
@given(c=PTR, r=PTR, K=I64, T=I64, L=I64, gamma=F32)
def test_reward_scan_answers_by_its_rules(c, r, K, T, L, gamma):
    Lb, lib = _abi()
    gamma = _f32(gamma)
    st_ = lib.dust_reward_scan(c, K, T, L, gamma, r, None)
    invalid = (None in (c, r) or K <= 0 or T <= 0 or L <= 0 or (T > 0 and L > 0 and T % L)
               or not _gamma_ok(gamma))
    if invalid:
        assert st_ == Lb.DUST_ERR_INVALID_ARG
    elif K * T > ELEMS_MAX:
        assert st_ == Lb.DUST_ERR_UNSUPPORTED
    else:
        assert st_ == HIP_FAIL


@ABI_SETTINGS
@given(g=PTR, X=PTR, G=PTR, xdt=ENUM, T=I64, N=I64, d=I64, ws=PTR, wsb=st.integers(0, 2**62))
def test_outer_sum_answers_by_its_rules(g, X, G, xdt, T, N, d, ws, wsb):
    Lb, lib = _abi()
    st_ = lib.dust_outer_sum(g, X, xdt, T, N, d, G, ws, wsb, None)
    invalid = None in (g, X, G) or xdt not in (0, 1) or T <= 0 or N <= 0 or d <= 0
    if invalid:
        assert st_ == Lb.DUST_ERR_INVALID_ARG
        return
    if T > T_MAX or N > WIDTH_MAX or d > WIDTH_MAX:
        assert st_ == Lb.DUST_ERR_UNSUPPORTED
        return
    assert st_ in (Lb.DUST_ERR_UNSUPPORTED, Lb.DUST_ERR_WORKSPACE, HIP_FAIL)
    need = lib.dust_outer_sum_workspace_size(T, N, d)
    assert need >= 256
    if st_ != Lb.DUST_ERR_UNSUPPORTED:
        assert (st_ == Lb.DUST_ERR_WORKSPACE) == (ws is None or wsb < need)


@ABI_SETTINGS
@given(T=I64, V=I64, d=I64, K=I64, gamma=F32, vocab=I64)
def test_size_queries_never_answer_zero(T, V, d, K, gamma, vocab):
    Lb, lib = _abi()
    gamma = _f32(gamma)
    assert lib.dust_head_workspace_size(T, V, d, K, gamma) >= 256
    assert lib.dust_linear_workspace_size(T, d, V, K, gamma) >= 256
    assert lib.dust_outer_sum_workspace_size(T, V, d) >= 256
    assert lib.dust_embedding_workspace_size(T, V, vocab) >= 256
    nb = lib.dust_embedding_noalloc_bytes(T, V, vocab)
    if T < 0 or V <= 0 or vocab <= 0 or T > T_MAX or V > WIDTH_MAX or vocab > 2**24:
        assert nb == 0


@ABI_SETTINGS
@given(code=st.integers(-2**31, 2**31 - 1))
def test_status_string_of_any_code(code):
    Lb, lib = _abi()
    s = lib.dust_status_string(code)
    assert s and s.startswith(b"DUST_")
    if code not in range(6):
        assert s == b"DUST_ERR_UNKNOWN"
