"""Each GPU stage of the estimator against the oracle (paper digest, section 2.2;
laoyaoba analysis, mechanism section), at sizes that span several tiles and
leave ragged tails.

Tolerances: per-draw losses |error| <= 2e-4 nats (fp32 logsumexp of ~6-nat
losses over up to 16k terms); centring and the scan within fp32 rounding
(relative L2 <= 1e-5; gamma = 0 is bit-exact); error estimate and outer product
relative L2 <= 1e-3 and cosine >= 0.99999, row by row and element by element
(util.assert_rows, util.assert_elementwise)."""
import numpy as np
import pytest

import oracle
from activation_perturbation_estimator_amd import synth
from util import (G_HAT_TERM_TOL, G_W_RSS_TOL, assert_elementwise, assert_parity, assert_rows,
                  gw_rss_scale, need_gpu, rel_l2)

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
                                   (2, 8200, 4100), (2, 2046, 1023), (3, 9000, 9),
                                   # one segment per tile, and segments longer than a
                                   # tile (8192): carried from tile to tile, with a
                                   # ragged first tile, vectorised or not
                                   (2, 16384, 8192), (2, 20000, 10000), (2, 16388, 8194),
                                   (1, 17001, 17001)])
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
    ref, sc = oracle.linear_rows(c, L, N, sigma, gamma, seed, list(range(T)), stream,
                                 with_scale=True)
    got = g.cpu().numpy()
    assert_parity(got, ref, "g_hat")
    assert_rows(got, ref, "g_hat rows")
    assert_elementwise(got, ref, sc, "g_hat elements", G_HAT_TERM_TOL)


def _check_outer(G, ref, g, X64):
    """G_W = g^T X: the parity bar on the whole array, and every element within
    G_W_RSS_TOL of its root-sum-square scale (the fp16 operands' error grows
    with that scale, not with the element: a row whose sums cancel keeps the
    same absolute error, so no per-row relative bar applies to G_W)."""
    assert_parity(G, ref, "G_W")
    assert_elementwise(G, ref, gw_rss_scale(g, X64), "G_W elements", G_W_RSS_TOL,
                       atol=1e-6 * float(np.abs(ref).max()))


def test_error_estimate_draw_ranges():
    """dust_error_estimate over draws [0, k) and [k, K) of a population of K
    adds up to the call over [0, K)."""
    dust = need_gpu()
    import torch
    K, T, N, k = 30, 40, 520, 11
    r = torch.from_numpy(np.random.default_rng(3).standard_normal((K, T)).astype(np.float32) * 0.03)
    full = dust.error_estimate(_cuda(r), N=N, sigma=0.02, seed=4, stream=1)
    a = dust.error_estimate(_cuda(r[:k]), N=N, sigma=0.02, seed=4, stream=1, K_total=K)
    b = dust.error_estimate(_cuda(r[k:]), N=N, sigma=0.02, seed=4, stream=1, draw0=k, K_total=K)
    torch.cuda.synchronize()
    ref, sc = oracle.linear_rows(r.double().numpy(), T, N, 0.02, 0.0, 4, list(range(T)), 1,
                                 with_scale=True)
    for got, what in ((full.cpu().numpy(), "whole"),
                      (a.cpu().double().numpy() + b.cpu().double().numpy(), "two ranges")):
        assert_parity(got, ref, what)
        assert_elementwise(got, ref, sc, what, G_HAT_TERM_TOL)


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
    _check_outer(G.cpu().numpy(), ref, g, synth.to_f64(X))


@pytest.mark.parametrize("own_flag", [True, False])
def test_check_targets(own_flag):
    """With the library's own flag (NULL) or a caller's, which starts dirty."""
    dust = need_gpu()
    import torch
    flag = None if own_flag else torch.full((1,), 7, dtype=torch.int32, device="cuda")
    y = torch.randint(0, 100, (1000,), dtype=torch.int32, device="cuda")
    assert dust.check_targets(y, 100, flag)
    y[517] = 100
    assert not dust.check_targets(y, 100, flag)
    y[517] = -1
    assert not dust.check_targets(y, 100, flag)
    y[517] = 5
    assert dust.check_targets(y, 100, flag)  # the flag is cleared by every call


@pytest.mark.parametrize("L,gamma", [(1024, 0.9), (1000, 0.9), (256, 1.0), (260, 0.5),
                                     (2048, 0.0)])
def test_reward_scan_unaligned(L, gamma):
    """c and r 4 bytes past a 16-byte boundary: the one-wave-per-segment scan
    then reads and writes element by element, through buffer resources bounded
    by the segment.  Nothing outside r is written."""
    dust = need_gpu()
    import torch
    K, T = 3, 4 * L
    c = np.random.default_rng(L).standard_normal((K, T)).astype(np.float32)
    cb = torch.zeros(K * T + 1, dtype=torch.float32, device="cuda")
    cb[1:] = torch.from_numpy(c.reshape(-1)).cuda()
    rb = torch.full((K * T + 2,), float("nan"), dtype=torch.float32, device="cuda")
    cv, rv = cb[1:].view(K, T), rb[1:K * T + 1].view(K, T)
    assert cv.data_ptr() % 16 == 4 and rv.data_ptr() % 16 == 4
    dust.reward_scan(cv, seq_len=L, gamma=gamma, out=rv)
    torch.cuda.synchronize()
    got = rb.cpu().numpy()
    assert np.isnan(got[0]) and np.isnan(got[-1])
    ref = oracle.reward_scan(c.astype(np.float64), L, gamma)
    if gamma == 0.0:
        assert np.array_equal(got[1:-1].reshape(K, T), c)
    else:
        assert rel_l2(got[1:-1].reshape(K, T), ref) <= 1e-5


def test_reward_scan_two_dimensional_grid():
    """2^24 + 1024 segments of 256 tokens (16 GiB per array): more one-wave
    workgroups than the launch puts in the grid's x dimension (2^24), so it
    adds a second one.  The input comes from torch's seeded generator on the
    device; segments sampled across the array, around the end of the first
    grid row and at the end, against the oracle."""
    dust = need_gpu()
    import torch
    L, gamma = 256, 0.9
    nseg = (1 << 24) + 1024
    T = nseg * L
    gen = torch.Generator(device="cuda").manual_seed(24)
    c = torch.randn((1, T), generator=gen, dtype=torch.float32, device="cuda")
    r = dust.reward_scan(c, seq_len=L, gamma=gamma)
    torch.cuda.synchronize()
    segs = np.concatenate([np.arange(4), np.arange((1 << 24) - 4, (1 << 24) + 8),
                           np.arange(nseg - 4, nseg),
                           np.random.default_rng(1).choice(nseg, 200, replace=False)])
    for sgi in segs:
        lo = int(sgi) * L
        cs = c[0, lo:lo + L].cpu().numpy().astype(np.float64).reshape(1, L)
        ref = oracle.reward_scan(cs, L, gamma)
        assert rel_l2(r[0, lo:lo + L].cpu().numpy().reshape(1, L), ref) <= 1e-5, sgi
    del c, r
    torch.cuda.empty_cache()


def test_reward_scan_many_short_segments():
    """K * T / L = 524288 (draw, sequence) segments of 2 tokens: a tile of the
    scan holds 1024 whole segments, so nearly every thread's elements span a
    segment end."""
    dust = need_gpu()
    import torch
    K, T, L = 4096, 256, 2
    c = np.random.default_rng(11).standard_normal((K, T)).astype(np.float32)
    r = dust.reward_scan(_cuda(torch.from_numpy(c)), seq_len=L, gamma=0.75)
    torch.cuda.synchronize()
    ref = oracle.reward_scan(c.astype(np.float64), L, 0.75)
    assert rel_l2(r.cpu().numpy(), ref) <= 1e-5


def test_outer_sum_many_tokens_fp32():
    """fp32 X over 65536 tokens (the operand pass writes 8 x 1 MiB token groups,
    many splits); d = 520 also leaves a ragged column tile."""
    dust = need_gpu()
    import torch
    T, N, d = 65536, 32, 520
    rng = np.random.default_rng(5)
    g = rng.standard_normal((T, N)).astype(np.float32)
    Xf = rng.standard_normal((T, d)).astype(np.float32)
    G = dust.outer_sum(_cuda(torch.from_numpy(g)), _cuda(torch.from_numpy(Xf)))
    torch.cuda.synchronize()
    ref = oracle.outer_sum(g.astype(np.float64), Xf.astype(np.float64))
    _check_outer(G.cpu().numpy(), ref, g, Xf.astype(np.float64))


@pytest.mark.parametrize("bf16", [True, False])
def test_outer_sum_exact_tokens(bf16):
    """Tokens whose |g| |x| range fits no power-of-two scaling into fp16 (very
    large and very small rows), zero rows, and non-finite values go through the
    exact fp32 pass; every other token through the fp16 matrix cores.  The
    result must match the fp64 product: NaN/inf exactly where the product has
    them, every finite element within the bounds."""
    dust = need_gpu()
    import torch
    T, N, d = 3000, 300, 136
    rng = np.random.default_rng(41)
    g = rng.standard_normal((T, N)).astype(np.float32)
    Xf = rng.standard_normal((T, d)).astype(np.float32)
    g[5] *= 1e18          # range far above fp16 for any split of the exponent
    g[1700] *= 1e-16      # far below
    Xf[2999] *= 1e-30     # x tiny, g normal: the product's range is too small
    g[77] = 0.0           # contributes nothing
    g[1234, 17] = np.nan  # NaN in one column of G_W
    Xf[2500, 3] = np.inf  # inf times g: +-inf in one column of G_W
    X = torch.from_numpy(Xf).to(torch.bfloat16) if bf16 else torch.from_numpy(Xf)
    G = dust.outer_sum(_cuda(torch.from_numpy(g)), _cuda(X)).cpu().numpy()
    X64 = synth.to_f64(X)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.outer_sum(g.astype(np.float64), X64)
    fin = np.isfinite(ref)
    assert not fin.all()
    assert np.array_equal(np.isnan(G), np.isnan(ref))
    assert np.array_equal(np.isinf(G), np.isinf(ref)) and (G[~fin & ~np.isnan(ref)] ==
                                                           ref[~fin & ~np.isnan(ref)]).all()
    gf = np.where(np.isfinite(g), g, 0.0).astype(np.float64)
    Xz = np.where(np.isfinite(X64), X64, 0.0)
    scale = gw_rss_scale(gf, Xz)
    err = np.abs(G[fin] - ref[fin])
    assert (err <= G_W_RSS_TOL * scale[fin] + 1e-6 * np.abs(ref[fin]).max()).all()
    assert rel_l2(G[fin], ref[fin]) <= 1e-3


def test_outer_sum_reads_nothing_past_its_operands():
    """The workspace filled with NaN before the call, and the caller's g and X
    as views of the first T rows of NaN-filled buffers: a read past the end of
    any operand (the tails of token splits, the padding tokens of the last
    group of eight, the last column tile) would put NaN into G_W.  Ragged T,
    several splits."""
    dust = need_gpu()
    import torch
    T, N, d = 9003, 264, 300
    rng = np.random.default_rng(43)
    g = rng.standard_normal((T, N)).astype(np.float32)
    Xf = rng.standard_normal((T, d)).astype(np.float32)
    for bf16 in (True, False):
        gbig = torch.full((T + 77, N), float("nan"), dtype=torch.float32, device="cuda")
        gbig[:T] = torch.from_numpy(g).cuda()
        X = torch.from_numpy(Xf).to(torch.bfloat16) if bf16 else torch.from_numpy(Xf)
        xbig = torch.full((T + 77, d), float("nan"), dtype=X.dtype, device="cuda")
        xbig[:T] = X.cuda()
        nbytes = dust.outer_sum_workspace_size(T, N, d)
        ws = torch.full((nbytes // 4 + 1024,), float("nan"), dtype=torch.float32, device="cuda")
        G = dust.outer_sum(gbig[:T], xbig[:T], workspace=ws.view(torch.uint8)).cpu().numpy()
        ref = oracle.outer_sum(g.astype(np.float64), synth.to_f64(X))
        assert np.isfinite(G).all()
        _check_outer(G, ref, g, synth.to_f64(X))


def test_composed_estimates_ignore_stale_workspace():
    """dust_head_estimate and dust_linear_estimate with their workspace filled
    with NaN: every byte the G_W pass reads is written by the same call."""
    dust = need_gpu()
    import torch
    z, y, X = synth.head_inputs(1003, 1000, 72, seed=44, bf16=True)
    ws = torch.full((dust.head_workspace_size(1003, 1000, 72, 9) // 4 + 64,), float("nan"),
                    device="cuda")
    g, G = dust.head_estimate(z.cuda(), y.cuda(), X.cuda(), sigma=0.05, K=9, seed=2,
                              workspace=ws.view(torch.uint8))
    g = g.cpu().numpy()
    G = G.cpu().numpy()
    assert np.isfinite(G).all()
    ref = g.astype(np.float64).T @ synth.to_f64(X)
    _check_outer(G, ref, g, synth.to_f64(X))
    Xl, c = synth.linear_inputs(2001, 40, 7, seed=45, c_seed=3, bf16=False)
    ws = torch.full((dust.linear_workspace_size(2001, 40, 200, 7, 0.5) // 4 + 64,),
                    float("nan"), device="cuda")
    g, G = dust.linear_estimate(Xl.cuda(), c.cuda(), N=200, sigma=0.01, gamma=0.5, seed=3,
                                seq_len=2001, workspace=ws.view(torch.uint8))
    g = g.cpu().numpy()
    G = G.cpu().numpy()
    assert np.isfinite(G).all()
    _check_outer(G, g.astype(np.float64).T @ synth.to_f64(Xl), g, synth.to_f64(Xl))
