"""Cosine-versus-population harness for the LM head.

The pages measure how well the estimate aligns with the backprop gradient as
the population grows and fit cos(K) = c_max / sqrt(1 + c / K) per layer type
(paper digest, section 4.2; linlog explainer, gradient-alignment section).
For the LM head the backprop gradient has a closed form, softmax(z) - onehot(y),
so the same measurement runs on any logits: this module times nothing and
trains nothing; it calls dust_head_estimate for each K, dust_ce_grad once, and
fits the law.  First-order analysis of the estimator predicts c = V + 1 and
c_max -> 1 as sigma -> 0 (noise covariance |g|^2 I + g g^T per draw).
"""
from __future__ import annotations

import math
from typing import Dict, Iterable

import numpy as np

from . import ce_grad, head_estimate


def fit_law(Ks, cos) -> Dict[str, float]:
    """Least-squares fit of cos(K) = c_max / sqrt(1 + c/K); returns c_max, c."""
    from scipy.optimize import curve_fit
    Ks = np.asarray(Ks, dtype=np.float64)
    cos = np.asarray(cos, dtype=np.float64)
    (cmax, c), _ = curve_fit(lambda k, cm, cc: cm / np.sqrt(1.0 + cc / k), Ks, cos,
                             p0=(1.0, float(Ks.max()) / 8),
                             bounds=([0.0, 0.0], [2.0, np.inf]), maxfev=20000)
    resid = cos - cmax / np.sqrt(1.0 + c / Ks)
    return {"c_max": float(cmax), "c": float(c), "rmse": float(np.sqrt(np.mean(resid ** 2)))}


def cosine_sweep(logits, targets, X, Ks: Iterable[int], *, sigma: float, seed: int = 1,
                 seq_len=None) -> Dict[str, object]:
    """Per-token cosine of g_hat with softmax(z) - onehot(y) and cosine of G_W
    with (softmax - onehot)^T X, for each population K; plus the fitted law."""
    import torch
    g_exact = ce_grad(logits, targets).double()
    G_exact = g_exact.T @ X.double()
    out = {"K": [], "cos_token_mean": [], "cos_token_se": [], "cos_GW": []}
    T = logits.shape[0]
    for K in Ks:
        g, G = head_estimate(logits, targets, X, sigma=sigma, K=int(K), gamma=0.0, seed=seed,
                             seq_len=seq_len)
        gd = g.double()
        cos = (gd * g_exact).sum(1) / (gd.norm(dim=1) * g_exact.norm(dim=1))
        cw = float((G.double() * G_exact).sum() / (G.double().norm() * G_exact.norm()))
        out["K"].append(int(K))
        out["cos_token_mean"].append(float(cos.mean()))
        out["cos_token_se"].append(float(cos.std() / math.sqrt(T)))
        out["cos_GW"].append(cw)
        torch.cuda.synchronize()
    out["fit_token"] = fit_law(out["K"], out["cos_token_mean"])
    V = logits.shape[1]
    out["first_order_c"] = V + 1
    return out
