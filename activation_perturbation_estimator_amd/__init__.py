"""libdust: the Dust virtual-population gradient estimator on MI355X (gfx950).

Thin torch-facing binding of the C ABI in ``include/dust.h``.  Each function
checks dtypes and shapes, allocates outputs (and the call's workspace) with
torch on the tensors' device, and calls the library on torch's current stream.
Every step of the estimator runs in libdust's HIP kernels; there is no CPU
path, and a missing library raises.

The method ("Dust: Pretraining Transformers Without Backpropagation", Q Labs),
as the pages about it state it (HN-mirror digest of the paper, section 2.2):
a linear layer's output y_t is jittered to y_t + sigma a_t for every token and
draw; token s scores a draw by its centred loss decrease c_s; the reward is
r_t = sum_{s>=t} gamma^(s-t) c_s inside the sequence; the output-error estimate
is g_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i); the weight gradient is
G_W = sum_t g_t x_t^T.  The LM head is perturbed on its cached logits and only
the cross-entropy is recomputed (laoyaoba analysis, mechanism section).
"""
from __future__ import annotations

from typing import Optional, Sequence

from . import _lib
from ._lib import (DUST_BF16, DUST_EMBEDDING_NOALLOC_BYTES, DUST_F32, DUST_N_MAX, DUST_SIGMA_MAX,
                   DUST_STAGE_EVENTS, DustError)

__all__ = [
    "head_estimate", "linear_estimate", "noise", "philox4x32_10", "head_losses", "centre",
    "reward_scan", "error_estimate", "outer_sum", "perturbed_linear", "embedding_grad",
    "embedding_grad_noalloc", "sgd_momentum_", "adam_", "ce_grad", "check_targets",
    "head_workspace_size",
    "linear_workspace_size", "outer_sum_workspace_size", "version", "DustError",
    "DUST_SIGMA_MAX", "DUST_N_MAX", "DUST_STAGE_EVENTS", "DUST_EMBEDDING_NOALLOC_BYTES",
]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DUST_F32
    if t.dtype == torch.bfloat16:
        return DUST_BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _expect(t, name: str, shape=None, dtypes=None, device=None) -> None:
    """Shape, dtype and device of a tensor the library reads or writes: the C
    ABI takes bare pointers, so a wrong-sized buffer must be refused here."""
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtypes is not None:
        dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
        if t.dtype not in dtypes:
            raise TypeError(f"{name} must be {' or '.join(map(str, dtypes))}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _f32():
    return _torch().float32


def _fp():
    torch = _torch()
    return (torch.float32, torch.bfloat16)


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _events(stage_events) -> Optional[object]:
    if stage_events is None:
        return None
    import ctypes
    if len(stage_events) != DUST_STAGE_EVENTS:
        raise ValueError(f"stage_events needs {DUST_STAGE_EVENTS} events")
    arr = (ctypes.c_void_p * DUST_STAGE_EVENTS)()
    for k, ev in enumerate(stage_events):  # None: that stage boundary is not recorded
        if ev is not None:
            arr[k] = int(ev.cuda_event) if hasattr(ev, "cuda_event") else int(ev)
    return arr


def _workspace(nbytes: int, device, workspace):
    torch = _torch()
    if workspace is not None:
        _expect(workspace, "workspace", device=device)
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _outputs(out, shapes, device, names):
    """Preallocated outputs (float32, exact shapes, on `device`), or fresh ones."""
    torch = _torch()
    if out is None:
        return tuple(torch.empty(sh, dtype=torch.float32, device=device) for sh in shapes)
    out = (out,) if len(shapes) == 1 and not isinstance(out, (tuple, list)) else tuple(out)
    if len(out) != len(shapes):
        raise ValueError(f"out must hold {len(shapes)} tensors")
    for o, sh, nm in zip(out, shapes, names):
        _expect(o, nm, sh, _f32(), device)
    return out


def version() -> str:
    return _lib.load().dust_version().decode()


def head_workspace_size(T: int, V: int, d: int, K: int, gamma: float = 0.0) -> int:
    return int(_lib.load().dust_head_workspace_size(T, V, d, K, gamma))


def linear_workspace_size(T: int, d_in: int, N: int, K: int, gamma: float = 0.0) -> int:
    return int(_lib.load().dust_linear_workspace_size(T, d_in, N, K, gamma))


def outer_sum_workspace_size(T: int, N: int, d: int) -> int:
    return int(_lib.load().dust_outer_sum_workspace_size(T, N, d))


def head_estimate(logits, targets, X, *, sigma: float, K: int, gamma: float = 0.0,
                  seed: int = 1, seq_len: Optional[int] = None, stream: int = 0,
                  return_losses: bool = False, stage_events: Optional[Sequence] = None,
                  workspace=None, out=None):
    """LM-head estimator on cached logits.

    logits [T,V] (f32/bf16), targets [T] int32, X [T,d] (f32/bf16), all on one
    GPU.  Returns (g_hat [T,V] f32, G_W [V,d] f32) and, with return_losses,
    the per-draw losses [K,T].  ``out`` may pass preallocated (g_hat, G_W).
    ``stage_events``: DUST_STAGE_EVENTS torch.cuda.Event objects (or None for a
    boundary that is not to be recorded) marking the stages on the stream."""
    torch = _torch()
    T, V = logits.shape
    d = X.shape[1]
    dev = logits.device
    _expect(logits, "logits", dtypes=_fp())
    _expect(targets, "targets", (T,), torch.int32, dev)
    _expect(X, "X", (T, d), _fp(), dev)
    L = T if seq_len is None else int(seq_len)
    g, G = _outputs(out, [(T, V), (V, d)], dev, ["g_hat", "G_W"])
    lib = _lib.load()
    losses = torch.empty((K, T), dtype=torch.float32, device=dev) if return_losses else None
    nbytes = lib.dust_head_workspace_size(T, V, d, K, gamma)
    ws = _workspace(nbytes, dev, workspace)
    st = lib.dust_head_estimate(
        _dev(logits, "logits"), _dtype_code(logits), _dev(targets, "targets"), _dev(X, "X"),
        _dtype_code(X), T, V, d, L, float(sigma), int(K), float(gamma), int(seed), int(stream),
        _dev(g, "g_hat"), _dev(G, "G_W"), losses.data_ptr() if losses is not None else None,
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev), _events(stage_events))
    _lib.check("dust_head_estimate", st)
    return (g, G, losses) if return_losses else (g, G)


def linear_estimate(X, c, *, N: int, sigma: float, gamma: float = 0.0, seed: int = 1,
                    seq_len: Optional[int] = None, stream: int = 0, draw0: int = 0,
                    K_total: Optional[int] = None, stage_events: Optional[Sequence] = None,
                    workspace=None, out=None):
    """Hidden linear layer: X [T,d_in] (f32/bf16), caller-centred loss decreases
    c [K,T] f32 measured with dust noise (seed, stream, draws draw0..draw0+K-1)
    of width N, normalised by a population of K_total draws (default K), so
    that calls over consecutive draw ranges add up.
    Returns (g_hat [T,N] f32, G_W [N,d_in] f32)."""
    T, d_in = X.shape
    K = c.shape[0]
    dev = X.device
    _expect(X, "X", dtypes=_fp())
    _expect(c, "c", (K, T), _f32(), dev)
    L = T if seq_len is None else int(seq_len)
    g, G = _outputs(out, [(T, N), (N, d_in)], dev, ["g_hat", "G_W"])
    lib = _lib.load()
    nbytes = lib.dust_linear_workspace_size(T, d_in, N, K, gamma)
    ws = _workspace(nbytes, dev, workspace)
    st = lib.dust_linear_estimate(
        _dev(X, "X"), _dtype_code(X), _dev(c, "c"), T, d_in, int(N), L, float(sigma), int(K),
        float(gamma), int(seed), int(stream), int(draw0), int(K if K_total is None else K_total),
        _dev(g, "g_hat"), _dev(G, "G_W"), ws.data_ptr(),
        ws.numel() * ws.element_size(), _stream(dev), _events(stage_events))
    _lib.check("dust_linear_estimate", st)
    return g, G


def noise(*, seed: int, stream: int = 0, draw0: int = 0, ndraw: int, T: int, N: int,
          device="cuda"):
    """a[k,t,n] = a^(draw0+k)_t[n] as float32 [ndraw,T,N] on `device`."""
    torch = _torch()
    out = torch.empty((ndraw, T, N), dtype=torch.float32, device=device)
    st = _lib.load().dust_noise(int(seed), int(stream), int(draw0), int(ndraw), int(T), int(N),
                                out.data_ptr(), _stream(out.device))
    _lib.check("dust_noise", st)
    return out


def philox4x32_10(seed: int, ctr):
    """Raw Philox4x32-10 blocks for counters ctr (int32/uint32 tensor [n,4] on GPU)."""
    torch = _torch()
    if ctr.dim() != 2 or ctr.shape[1] != 4 or ctr.dtype not in (torch.int32, torch.uint32):
        raise ValueError("ctr must be an int32 or uint32 [n,4] tensor")
    out = torch.empty_like(ctr)
    st = _lib.load().dust_philox4x32_10(int(seed), _dev(ctr, "ctr"), out.data_ptr(),
                                        ctr.shape[0], _stream(ctr.device))
    _lib.check("dust_philox4x32_10", st)
    return out


def head_losses(logits, targets, *, sigma: float, K: int, seed: int = 1, stream: int = 0):
    """Per-draw perturbed LM-head losses [K,T] f32."""
    torch = _torch()
    T, V = logits.shape
    _expect(logits, "logits", dtypes=_fp())
    _expect(targets, "targets", (T,), torch.int32, logits.device)
    out = torch.empty((K, T), dtype=torch.float32, device=logits.device)
    st = _lib.load().dust_head_losses(_dev(logits, "logits"), _dtype_code(logits),
                                      _dev(targets, "targets"), T, V, float(sigma), int(K),
                                      int(seed), int(stream), out.data_ptr(),
                                      _stream(logits.device))
    _lib.check("dust_head_losses", st)
    return out


def centre(x, out=None):
    """c[i,t] = mean_j x[j,t] - x[i,t] for per-draw losses x [K,T] f32."""
    K, T = x.shape
    _expect(x, "x", dtypes=_f32())
    (c,) = _outputs(out, [(K, T)], x.device, ["out"])
    st = _lib.load().dust_centre(_dev(x, "x"), K, T, _dev(c, "c"), _stream(x.device))
    _lib.check("dust_centre", st)
    return c


def reward_scan(c, *, seq_len: int, gamma: float, out=None):
    """r = segmented reverse gamma-scan of c [K,T] f32."""
    K, T = c.shape
    _expect(c, "c", dtypes=_f32())
    (r,) = _outputs(out, [(K, T)], c.device, ["out"])
    st = _lib.load().dust_reward_scan(_dev(c, "c"), K, T, int(seq_len), float(gamma),
                                      _dev(r, "r"), _stream(c.device))
    _lib.check("dust_reward_scan", st)
    return r


def error_estimate(r, *, N: int, sigma: float, seed: int = 1, stream: int = 0, draw0: int = 0,
                   K_total: Optional[int] = None, out=None):
    """g_hat[t,n] = -(1/(K_total sigma)) sum_i r[i,t] a^(draw0+i)_t[n] with
    regenerated noise (K_total defaults to K = r.shape[0])."""
    K, T = r.shape
    _expect(r, "r", dtypes=_f32())
    (g,) = _outputs(out, [(T, int(N))], r.device, ["out"])
    st = _lib.load().dust_error_estimate(_dev(r, "r"), K, T, int(N), float(sigma), int(seed),
                                         int(stream), int(draw0),
                                         int(K if K_total is None else K_total), _dev(g, "g_hat"),
                                         _stream(r.device))
    _lib.check("dust_error_estimate", st)
    return g


def outer_sum(g_hat, X, out=None, workspace=None):
    """G_W = g_hat^T X (sum over tokens), fp32 [N,d]."""
    T, N = g_hat.shape
    d = X.shape[1]
    _expect(g_hat, "g_hat", dtypes=_f32())
    _expect(X, "X", (T, d), _fp(), g_hat.device)
    (G,) = _outputs(out, [(N, d)], g_hat.device, ["out"])
    lib = _lib.load()
    nbytes = lib.dust_outer_sum_workspace_size(T, N, d)
    ws = _workspace(nbytes, g_hat.device, workspace)
    st = lib.dust_outer_sum(_dev(g_hat, "g_hat"), _dev(X, "X"), _dtype_code(X), T, N, d,
                            _dev(G, "G_W"), ws.data_ptr(), ws.numel() * ws.element_size(),
                            _stream(g_hat.device))
    _lib.check("dust_outer_sum", st)
    return G


def perturbed_linear(X, W, *, sigma: float, seed: int = 1, stream: int = 0, draw0: int = 0,
                     ndraw: int = 1, out=None):
    """Y[k] = X W^T + sigma a^(draw0+k) as float32 [ndraw, T, N]: the caller's
    perturbed forward, with the noise dust_linear_estimate regenerates."""
    T, d = X.shape
    N = W.shape[0]
    _expect(X, "X", dtypes=_fp())
    _expect(W, "W", (N, d), X.dtype, X.device)
    (Y,) = _outputs(out, [(int(ndraw), T, N)], X.device, ["out"])
    st = _lib.load().dust_perturbed_linear(_dev(X, "X"), _dev(W, "W"), _dtype_code(X), T, d, N,
                                           float(sigma), int(seed), int(stream), int(draw0),
                                           int(ndraw), _dev(Y, "Y"), _stream(X.device))
    _lib.check("dust_perturbed_linear", st)
    return Y


def embedding_grad(ids, g_hat, vocab: int, out=None, workspace=None):
    """G_E[v] = sum_{t: ids[t] = v} g_hat[t] as float32 [vocab, N] (one-hot input:
    the outer product is a scatter-add; deterministic order)."""
    torch = _torch()
    T, N = g_hat.shape
    _expect(g_hat, "g_hat", dtypes=_f32())
    _expect(ids, "ids", (T,), torch.int32, g_hat.device)
    (G,) = _outputs(out, [(int(vocab), N)], g_hat.device, ["out"])
    lib = _lib.load()
    ws = _workspace(lib.dust_embedding_workspace_size(T, N, int(vocab)), g_hat.device, workspace)
    st = lib.dust_embedding_grad(_dev(ids, "ids"), _dev(g_hat, "g_hat"), T, N, int(vocab),
                                 _dev(G, "G_E"), ws.data_ptr(), ws.numel() * ws.element_size(),
                                 _stream(g_hat.device))
    _lib.check("dust_embedding_grad", st)
    return G


def embedding_grad_noalloc(ids, g_hat, vocab: int, out=None):
    """embedding_grad without a workspace: the library's own fixed scratch
    (DUST_EMBEDDING_NOALLOC_BYTES per GPU), for callers that cannot allocate
    device memory.  ``out`` should be preallocated by such a caller."""
    torch = _torch()
    T, N = g_hat.shape
    _expect(g_hat, "g_hat", dtypes=_f32())
    _expect(ids, "ids", (T,), torch.int32, g_hat.device)
    (G,) = _outputs(out, [(int(vocab), N)], g_hat.device, ["out"])
    st = _lib.load().dust_embedding_grad_noalloc(_dev(ids, "ids"), _dev(g_hat, "g_hat"), T, N,
                                                 int(vocab), _dev(G, "G_E"),
                                                 _stream(g_hat.device))
    _lib.check("dust_embedding_grad_noalloc", st)
    return G


def sgd_momentum_(W, G, m, *, lr: float, momentum: float = 0.9, weight_decay: float = 0.0):
    """In place: m = momentum m + (G + wd W); W -= lr m (float32 tensors of one size)."""
    for t, nm in ((W, "W"), (G, "G"), (m, "m")):
        _expect(t, nm, W.shape, _f32(), W.device)
    st = _lib.load().dust_sgd_momentum(_dev(W, "W"), _dev(G, "G"), _dev(m, "m"), W.numel(),
                                       float(lr), float(momentum), float(weight_decay),
                                       _stream(W.device))
    _lib.check("dust_sgd_momentum", st)
    return W


def adam_(W, G, m, v, *, lr: float, step: int, beta1: float = 0.9, beta2: float = 0.999,
          eps: float = 1e-8, weight_decay: float = 0.0):
    """In place Adam step (bias-corrected, PyTorch semantics) on float32 tensors."""
    for t, nm in ((W, "W"), (G, "G"), (m, "m"), (v, "v")):
        _expect(t, nm, W.shape, _f32(), W.device)
    st = _lib.load().dust_adam(_dev(W, "W"), _dev(G, "G"), _dev(m, "m"), _dev(v, "v"), W.numel(),
                               float(lr), float(beta1), float(beta2), float(eps),
                               float(weight_decay), int(step), _stream(W.device))
    _lib.check("dust_adam", st)
    return W


def ce_grad(logits, targets, out=None):
    """softmax(z) - onehot(y) as float32 [T,V]: the closed-form LM-head gradient."""
    torch = _torch()
    T, V = logits.shape
    _expect(logits, "logits", dtypes=_fp())
    _expect(targets, "targets", (T,), torch.int32, logits.device)
    (o,) = _outputs(out, [(T, V)], logits.device, ["out"])
    st = _lib.load().dust_ce_grad(_dev(logits, "logits"), _dtype_code(logits),
                                  _dev(targets, "targets"), T, V, _dev(o, "out"),
                                  _stream(logits.device))
    _lib.check("dust_ce_grad", st)
    return o


def check_targets(targets, V: int, flag=None) -> bool:
    """True when 0 <= targets < V everywhere (waits for the device).  ``flag``:
    a device int32 tensor the call may overwrite, or None for the library's own."""
    torch = _torch()
    _expect(targets, "targets", dtypes=torch.int32)
    if flag is not None:
        _expect(flag, "flag", (1,), torch.int32, targets.device)
    st = _lib.load().dust_check_targets(_dev(targets, "targets"), targets.numel(), int(V),
                                        None if flag is None else flag.data_ptr(),
                                        _stream(targets.device))
    if st == _lib.DUST_ERR_TARGETS:
        return False
    _lib.check("dust_check_targets", st)
    return True
