"""Shared test helpers (comparison metrics, GPU gating, cross-check builds)."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "pins")
PIN_BUILD = os.path.join(ROOT, "_build", "pins")


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def cosine(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


# Parity bar on g_hat and G_W: relative L2 <= 1e-3 and cosine >= 0.99999,
# fp32 accumulation on the GPU against the fp64 oracle.
REL_L2_MAX = 1e-3
COS_MIN = 0.99999


def assert_parity(gpu, ref, what: str, rel=REL_L2_MAX, cos=COS_MIN):
    r = rel_l2(gpu, ref)
    c = cosine(gpu, ref)
    print(f"[parity] {what}: rel_l2={r:.3e} cos={c:.8f}", flush=True)
    assert r <= rel and c >= cos, f"{what}: rel_l2={r:.3e} cos={c:.8f}"


def assert_rows(gpu, ref, what: str, rel=REL_L2_MAX, cos=COS_MIN):
    """The parity bar row by row (one row = one token's g_hat): relative L2 and
    cosine of every row whose reference is not zero; rows whose reference is
    zero must be zero.  A fault confined to a few rows or columns of a large
    array cannot hide behind the whole-array norm."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    nr = np.linalg.norm(r, axis=1)
    ng = np.linalg.norm(g, axis=1)
    diff = np.linalg.norm(g - r, axis=1)
    zero = nr == 0
    assert np.all(diff[zero] == 0), f"{what}: rows {np.nonzero(zero & (diff > 0))[0][:8]} " \
        "should be zero"
    if (~zero).any():
        rr = diff[~zero] / nr[~zero]
        cc = (g * r).sum(1)[~zero] / np.maximum(ng[~zero] * nr[~zero], 1e-300)
        rows = np.nonzero(~zero)[0]
        i, j = int(np.argmax(rr)), int(np.argmin(cc))
        assert rr[i] <= rel and cc[j] >= cos, \
            f"{what}: worst row {rows[i]} rel_l2={rr[i]:.3e}, worst row {rows[j]} cos={cc[j]:.8f}"


def assert_elementwise(gpu, ref, scale, what: str, c: float, atol: float = 0.0):
    """|gpu - ref| <= c * scale + atol for every element, where `scale` is the
    size of what that element sums (computed from the oracle), so that a wrong,
    missing or extra term in any single element shows."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64)
    err = np.abs(g - r)
    bad = err > c * s + atol
    if bad.any():
        idx = np.unravel_index(int(np.argmax(np.where(bad, err / (c * s + atol + 1e-300), 0))),
                               err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of bound, worst at {idx}: "
                             f"|err|={err[idx]:.3e} bound={c * s[idx] + atol:.3e} "
                             f"ref={r[idx]:.3e}")


# g_hat: each element sums K terms r_i a_i / (K sigma); fp32 evaluation errs by
# ~1e-6 of the terms' magnitude sum_i |r_i a_i| / (K sigma), plus, since the
# rewards themselves are single precision (a loss change from a ratio of exp
# sums, a discounted scan), a floor of ~1e-7 of the token's largest reward on
# every term: the oracle's scale is (1/(K sigma)) sum_i (|r_i| + max_j |r_j|)
# |a_i|.  1e-4 of it is far above rounding and far below a wrong column, lane
# share or row.
G_HAT_TERM_TOL = 1e-4
# G_W from the composed calls: each element sums T products g_t x_t whose
# operands the matrix cores take rounded to 11 significant bits (relative error
# <= 2^-11 each, independent between tokens), so the error is a sum of
# independent terms with standard deviation <= 2^-11 sqrt(sum_t g^2 x^2) (fp32
# operands: both rounded, sqrt(2) more); 8 x 2^-11 of that root-sum-square is
# over 9 standard deviations.
G_W_RSS_TOL = 8 * 2.0 ** -11


def gw_rss_scale(g, X):
    """sqrt(sum_t g[t,n]^2 X[t,k]^2) for every element of G_W = g^T X."""
    g = np.asarray(g, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    return np.sqrt((g * g).T @ (X * X))


def assert_gw(G, g_ref, X, what="G_W"):
    """G_W against the fp64 product of the reference g_hat and X: the parity bar
    on the whole array, and element by element within G_W_RSS_TOL of each
    element's root-sum-square scale (plus 1e-6 of the largest entry)."""
    g_ref = np.asarray(g_ref, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    ref = g_ref.T @ X
    assert_parity(G, ref, what)
    assert_elementwise(G, ref, gw_rss_scale(g_ref, X), what, G_W_RSS_TOL,
                       atol=1e-6 * float(np.abs(ref).max()))


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import activation_perturbation_estimator_amd as dust
    dust._lib.load()  # a missing library must fail, not skip
    return dust


def pin_lib(name: str, compiler: list, extra: list):
    """Build (once) and load a test-only cross-check library from tests/pins."""
    os.makedirs(PIN_BUILD, exist_ok=True)
    src = os.path.join(PINS, name + ".cpp")
    so = os.path.join(PIN_BUILD, "lib" + name + ".so")
    if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        tmp = so + ".tmp%d" % os.getpid()
        subprocess.check_call(compiler + ["-O2", "-std=c++17", "-shared", "-fPIC", *extra, src,
                                          "-o", tmp], stderr=subprocess.DEVNULL)
        os.replace(tmp, so)
    return ctypes.CDLL(so)
