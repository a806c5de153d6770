"""fp64 CPU oracle of the Dust virtual-population gradient estimator.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product path (libdust and its Python
binding) never imports this package and shares no code with it.

The arithmetic lives in ``dust_oracle.c`` (plain C, double precision, libm);
this module only builds that file with gcc, loads it with ctypes and marshals
numpy arrays.  Every function states the passage of the pages it follows; the
pages are the web pages about "Dust: Pretraining Transformers Without
Backpropagation" (Q Labs).  The formulas are those of the HN-mirror digest of
the paper, section 2.2 (credit assignment).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dust_oracle.c")
_LIB = os.path.join(_HERE, "libdust_oracle.so")

_lib = None

_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_f64 = ctypes.c_double


def build(force: bool = True) -> str:
    """Compile dust_oracle.c into libdust_oracle.so with gcc (-O2, OpenMP)."""
    global _lib
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # DUST_ORACLE_LIB names another build of dust_oracle.c to load as it is
    # (the test suite's sanitizer build); by default the file next to the source.
    path = os.environ.get("DUST_ORACLE_LIB")
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    lib.oracle_philox_batch.argtypes = [_u64, _u32p, _u32p, _i64]
    lib.oracle_philox_batch.restype = None
    lib.oracle_uniform_batch.argtypes = [_u32p, _f64p, _i64]
    lib.oracle_uniform_batch.restype = None
    lib.oracle_angle_batch.argtypes = [_u32p, _f64p, _i64]
    lib.oracle_angle_batch.restype = None
    lib.oracle_noise.argtypes = [_u64, _u32, _i64, _i64, _i64, _i64, _f64p]
    lib.oracle_noise.restype = None
    lib.oracle_reward_scan.argtypes = [_f64p, _i64, _i64, _i64, _f64, _f64p]
    lib.oracle_reward_scan.restype = None
    lib.oracle_outer_sum.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _f64p]
    lib.oracle_outer_sum.restype = None
    opt = ctypes.c_void_p
    lib.oracle_head_estimate.argtypes = [_f64p, _i32p, _f64p, _i64, _i64, _i64, _i64,
                                         _f64, _i64, _f64, _u64, _u32,
                                         _f64p, _f64p, opt, opt, opt, opt, opt]
    lib.oracle_head_estimate.restype = ctypes.c_int
    lib.oracle_head_rows.argtypes = [_f64p, _i32p, _i64, _i64, _i64, _f64, _i64, _f64,
                                     _u64, _u32, _i64p, _i64, _f64p, opt, opt]
    lib.oracle_head_rows.restype = ctypes.c_int
    lib.oracle_linear_estimate.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _i64, _f64,
                                           _i64, _f64, _u64, _u32, _f64p, _f64p, opt, opt]
    lib.oracle_linear_estimate.restype = ctypes.c_int
    lib.oracle_linear_rows.argtypes = [_f64p, _i64, _i64, _i64, _f64, _i64, _f64, _u64,
                                       _u32, _i64p, _i64, _f64p, opt]
    lib.oracle_linear_rows.restype = ctypes.c_int
    lib.oracle_perturbed_linear.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _f64, _u64, _u32,
                                            _i64, _i64, _f64p]
    lib.oracle_perturbed_linear.restype = ctypes.c_int
    lib.oracle_embedding_grad.argtypes = [_i32p, _f64p, _i64, _i64, _i64, _f64p]
    lib.oracle_embedding_grad.restype = ctypes.c_int
    lib.oracle_sgd_momentum.argtypes = [_f64p, _f64p, _f64p, _i64, _f64, _f64, _f64]
    lib.oracle_sgd_momentum.restype = None
    lib.oracle_adam.argtypes = [_f64p, _f64p, _f64p, _f64p, _i64, _f64, _f64, _f64, _f64, _f64,
                                _i64]
    lib.oracle_adam.restype = None
    lib.oracle_ce_grad.argtypes = [_f64p, _i32p, _i64, _i64, _f64p]
    lib.oracle_ce_grad.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64c(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def philox4x32_10(seed: int, ctr) -> np.ndarray:
    """Raw Philox4x32-10 blocks (Salmon et al., SC'11) for counters ctr [n,4]."""
    ctr = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(-1, 4))
    out = np.empty_like(ctr)
    _load().oracle_philox_batch(int(seed) & (2**64 - 1), ctr, out, ctr.shape[0])
    return out


def uniform(x) -> np.ndarray:
    """u = ((x >> 9) + 1/2) / 2^23 for uint32 words x."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.uint32)).ravel()
    u = np.empty(x.shape[0], dtype=np.float64)
    _load().oracle_uniform_batch(x, u, x.shape[0])
    return u


def angle(x) -> np.ndarray:
    """v = (x >> 9) / 2^23 for uint32 words x: the Box-Muller angle in revolutions."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.uint32)).ravel()
    v = np.empty(x.shape[0], dtype=np.float64)
    _load().oracle_angle_batch(x, v, x.shape[0])
    return v


def noise(seed: int, stream: int, draw0: int, ndraw: int, T: int, N: int) -> np.ndarray:
    """a[k, t, n] for draws draw0..draw0+ndraw-1: the standard-normal noise of the
    pages (laoyaoba analysis, mechanism section; linlog explainer, virtual
    population section) under the Philox + Box-Muller convention."""
    out = np.empty((ndraw, T, N), dtype=np.float64)
    _load().oracle_noise(int(seed), int(stream), int(draw0), int(ndraw), int(T), int(N), out)
    return out


def reward_scan(c, L: int, gamma: float) -> np.ndarray:
    """r_t = sum_{s>=t, same sequence} gamma^(s-t) c_s (paper digest, section 2.2)."""
    c = _f64c(c)
    K, T = c.shape
    if L <= 0 or T % L != 0:
        raise ValueError("T must be a multiple of the sequence length L")
    r = np.empty_like(c)
    _load().oracle_reward_scan(c, K, T, int(L), float(gamma), r)
    return r


def outer_sum(g, X) -> np.ndarray:
    """G_W = sum_t g_t x_t^T (paper digest, section 2.2)."""
    g = _f64c(g)
    X = _f64c(X)
    T, N = g.shape
    d = X.shape[1]
    G = np.empty((N, d), dtype=np.float64)
    _load().oracle_outer_sum(g, X, T, N, d, G)
    return G


def head_estimate(logits, targets, X, seq_len: int, sigma: float, K: int, gamma: float,
                  seed: int, stream: int = 0, diagnostics: bool = False):
    """LM-head estimator: noise on cached logits, CE recomputed per draw
    (laoyaoba analysis, mechanism section; linlog explainer, virtual population
    section), then the credit assignment of the paper digest, section 2.2.

    Returns (g_hat [T,V], G_W [V,d]) and, with diagnostics, a dict with
    ell [K,T], c [K,T], r [K,T], ell0 [T] and g_scale [T,V], the scale of the
    rounding error of each element of g_hat: (1/(K sigma)) sum_i (|r_i| +
    max_j |r_j|) |a_i|, the magnitude of its terms plus the same with every
    reward replaced by the token's largest."""
    z = _f64c(logits)
    y = np.ascontiguousarray(np.asarray(targets, dtype=np.int32))
    Xd = _f64c(X)
    T, V = z.shape
    d = Xd.shape[1]
    g = np.empty((T, V), dtype=np.float64)
    G = np.empty((V, d), dtype=np.float64)
    diag = None
    if diagnostics:
        diag = {"ell": np.empty((K, T)), "c": np.empty((K, T)), "r": np.empty((K, T)),
                "ell0": np.empty(T), "g_scale": np.empty((T, V))}
    rc = _load().oracle_head_estimate(
        z, y, Xd, T, V, d, int(seq_len), float(sigma), int(K), float(gamma),
        int(seed), int(stream), g, G,
        _ptr(diag["ell"]) if diag else None, _ptr(diag["c"]) if diag else None,
        _ptr(diag["r"]) if diag else None, _ptr(diag["ell0"]) if diag else None,
        _ptr(diag["g_scale"]) if diag else None)
    if rc != 0:
        raise ValueError("oracle_head_estimate rejected its arguments")
    return (g, G, diag) if diagnostics else (g, G)


def head_rows(logits, targets, seq_len: int, sigma: float, K: int, gamma: float,
              seed: int, tokens, stream: int = 0, with_losses: bool = False,
              with_scale: bool = False):
    """Error-estimate rows g_hat[tokens, :] of the LM-head estimator, computed
    token by token (same steps as head_estimate).  With with_losses the
    per-draw losses [K, n] follow; with with_scale the error scales
    (1/(K sigma)) sum_i |r_i a_i| of the same rows [n, V] come last."""
    z = _f64c(logits)
    y = np.ascontiguousarray(np.asarray(targets, dtype=np.int32))
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    T, V = z.shape
    rows = np.empty((tok.shape[0], V), dtype=np.float64)
    ell = np.empty((K, tok.shape[0]), dtype=np.float64) if with_losses else None
    scale = np.empty_like(rows) if with_scale else None
    rc = _load().oracle_head_rows(z, y, T, V, int(seq_len), float(sigma), int(K),
                                  float(gamma), int(seed), int(stream), tok, tok.shape[0],
                                  rows, _ptr(ell), _ptr(scale))
    if rc != 0:
        raise ValueError("oracle_head_rows rejected its arguments")
    out = (rows,) + ((ell,) if with_losses else ()) + ((scale,) if with_scale else ())
    return out if len(out) > 1 else rows


def linear_estimate(X, c, seq_len: int, N: int, sigma: float, gamma: float, seed: int,
                    stream: int = 0, with_r: bool = False, with_scale: bool = False):
    """Hidden linear layer: caller's centred loss decreases c [K,T] -> reward scan,
    error estimate and outer product (paper digest, section 2.2).  Returns
    (g_hat, G_W), then r [K,T] with with_r, then the error scales of g_hat
    [T,N] with with_scale."""
    Xd = _f64c(X)
    cd = _f64c(c)
    K, T = cd.shape
    d_in = Xd.shape[1]
    g = np.empty((T, N), dtype=np.float64)
    G = np.empty((N, d_in), dtype=np.float64)
    r = np.empty((K, T), dtype=np.float64) if with_r else None
    scale = np.empty_like(g) if with_scale else None
    rc = _load().oracle_linear_estimate(Xd, cd, T, d_in, int(N), int(seq_len), float(sigma),
                                        int(K), float(gamma), int(seed), int(stream), g, G,
                                        _ptr(r), _ptr(scale))
    if rc != 0:
        raise ValueError("oracle_linear_estimate rejected its arguments")
    return (g, G) + ((r,) if with_r else ()) + ((scale,) if with_scale else ())


def linear_rows(c, seq_len: int, N: int, sigma: float, gamma: float, seed: int, tokens,
                stream: int = 0, with_scale: bool = False):
    """Error-estimate rows g_hat[tokens, :] of the linear-layer estimator (and,
    with with_scale, the error scales of the same rows)."""
    cd = _f64c(c)
    K, T = cd.shape
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    rows = np.empty((tok.shape[0], N), dtype=np.float64)
    scale = np.empty_like(rows) if with_scale else None
    rc = _load().oracle_linear_rows(cd, T, int(N), int(seq_len), float(sigma), int(K),
                                    float(gamma), int(seed), int(stream), tok, tok.shape[0],
                                    rows, _ptr(scale))
    if rc != 0:
        raise ValueError("oracle_linear_rows rejected its arguments")
    return (rows, scale) if with_scale else rows


def perturbed_linear(X, W, sigma: float, seed: int, stream: int = 0, draw0: int = 0,
                     ndraw: int = 1) -> np.ndarray:
    """Y[k] = X W^T + sigma a^(draw0+k): the perturbed forward of a hidden linear
    layer (paper digest, sections 2 and 2.1)."""
    Xd = _f64c(X)
    Wd = _f64c(W)
    T, d = Xd.shape
    N = Wd.shape[0]
    Y = np.empty((ndraw, T, N), dtype=np.float64)
    rc = _load().oracle_perturbed_linear(Xd, Wd, T, d, N, float(sigma), int(seed), int(stream),
                                         int(draw0), int(ndraw), Y)
    if rc != 0:
        raise ValueError("oracle_perturbed_linear rejected its arguments")
    return Y


def embedding_grad(ids, g, vocab: int) -> np.ndarray:
    """G_E[v] = sum_{t: ids[t]=v} g[t] (paper digest, section 2.2: one-hot input)."""
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    gd = _f64c(g)
    T, N = gd.shape
    GE = np.empty((vocab, N), dtype=np.float64)
    if _load().oracle_embedding_grad(ids, gd, T, N, int(vocab), GE) != 0:
        raise ValueError("oracle_embedding_grad rejected its arguments")
    return GE


def sgd_momentum(W, G, m, lr: float, momentum: float, weight_decay: float = 0.0):
    """One SGD-with-momentum step; returns (W, m) as new fp64 arrays."""
    W = _f64c(W).copy()
    m = _f64c(m).copy()
    _load().oracle_sgd_momentum(W.ravel(), _f64c(G).ravel(), m.ravel(), W.size, float(lr),
                                float(momentum), float(weight_decay))
    return W, m


def adam(W, G, m, v, lr: float, step: int, beta1: float = 0.9, beta2: float = 0.999,
         eps: float = 1e-8, weight_decay: float = 0.0):
    """One bias-corrected Adam step; returns (W, m, v) as new fp64 arrays."""
    W = _f64c(W).copy()
    m = _f64c(m).copy()
    v = _f64c(v).copy()
    _load().oracle_adam(W.ravel(), _f64c(G).ravel(), m.ravel(), v.ravel(), W.size, float(lr),
                        float(beta1), float(beta2), float(eps), float(weight_decay), int(step))
    return W, m, v


def ce_grad(logits, targets) -> np.ndarray:
    """softmax(z_t) - onehot(y_t) in fp64."""
    z = _f64c(logits)
    y = np.ascontiguousarray(np.asarray(targets, dtype=np.int32))
    T, V = z.shape
    out = np.empty((T, V), dtype=np.float64)
    _load().oracle_ce_grad(z, y, T, V, out)
    return out
